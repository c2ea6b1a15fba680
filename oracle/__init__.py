"""fp64 CPU oracle for the Gated DeltaNet forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it and it
shares no code with the GPU library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, token-by-token; the
definition and its source passage are in that file's header).  This module
only compiles it with gcc and marshals numpy arrays through ctypes.

Parity pins: ``tests/test_oracle_pins.py`` and ``tests/golden/``.

``attn_sink_window`` (from ``attention.py``) is the oracle of the softmax
attention block with a sink chunk and a recent window; ``gdn_framewise``
(from ``framewise.py``) that of frame-wise Gated DeltaNet with a normalised
readout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .attention import attn_sink_window  # noqa: F401
from .framewise import gdn_framewise  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

DEFAULT_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                       ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                       ctypes.c_long, ctypes.c_long,
                                       ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_int]
        lib.gdn_oracle_scan.restype = ctypes.c_int
        lib.gdn_oracle_scan.argtypes = lib.gdn_oracle_fwd.argtypes[:-1] + [ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_gates.restype = None
        lib.gdn_oracle_gates.argtypes = [dp, dp, dp, dp, ctypes.c_long]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gates(a, b):
    """alpha = exp(-softplus(a)), beta = sigmoid(b) in fp64 (gdn_oracle_gates)."""
    a, b = _f64(a), _f64(b)
    assert a.shape == b.shape
    alpha = np.empty_like(a)
    beta = np.empty_like(b)
    _load().gdn_oracle_gates(_ptr(a), _ptr(b), _ptr(alpha), _ptr(beta), a.size)
    return alpha, beta


def gdn_fwd(q, k, v, alpha, beta, state_in=None, *, qk_l2norm=True, scale=1.0,
            eps=DEFAULT_EPS, nthreads=0, want_state=True, gate_logits=False, out_gate=None,
            reverse=False):
    """Token-by-token fp64 gated delta rule.

    Shapes: q, k [B,H,T,dk]; v [B,H,T,dv]; alpha, beta [B,H,T];
    state_in [B,H,dk,dv] or None (zero state).  Inputs of any float dtype are
    converted to fp64 exactly (bf16/fp16/fp32 all embed in fp64).
    gate_logits: alpha, beta hold logits a, b (see gates()).  out_gate
    [B,H,T,dv]: the outputs are multiplied by it elementwise.  reverse: the
    backward scan (tokens visited from T-1 down to 0; gdn_oracle_scan).
    Returns (out [B,H,T,dv] fp64, state_out [B,H,dk,dv] fp64 or None).
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    if gate_logits:
        alpha, beta = gates(alpha, beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, T) and beta.shape == (B, H, T)
    s_in = None
    if state_in is not None:
        s_in = _f64(state_in)
        assert s_in.shape == (B, H, dk, dv)
    out = np.empty((B, H, T, dv), dtype=np.float64)
    s_out = np.empty((B, H, dk, dv), dtype=np.float64) if want_state else None
    rc = _load().gdn_oracle_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(s_in), _ptr(out), _ptr(s_out),
                                 B, H, T, dk, dv, 1 if qk_l2norm else 0,
                                 float(scale), float(eps), 1 if reverse else 0, int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_fwd failed with code %d" % rc)
    if out_gate is not None:
        g = _f64(out_gate)
        assert g.shape == out.shape
        out = out * g
    return out, s_out


def gdn_bidir(q, k, v, alpha, beta, state_in=None, *, qk_l2norm=True, scale=1.0,
              eps=DEFAULT_EPS, nthreads=0, gate_logits=False, out_gate=None):
    """Bidirectional GDN over one streaming chunk (SANA-Streaming section 4.1:
    forward scan from the previous cache, backward scan within the chunk;
    section 2.3: the two histories are combined for the output):
    out = o^f + o^b, with o^f the forward scan from state_in and o^b the
    backward scan from a zero state; then the output gate.  Returns
    (out, the forward scan's final state)."""
    of, sf = gdn_fwd(q, k, v, alpha, beta, state_in, qk_l2norm=qk_l2norm, scale=scale, eps=eps,
                     nthreads=nthreads, gate_logits=gate_logits)
    ob, _ = gdn_fwd(q, k, v, alpha, beta, None, qk_l2norm=qk_l2norm, scale=scale, eps=eps,
                    nthreads=nthreads, want_state=False, gate_logits=gate_logits, reverse=True)
    out = of + ob
    if out_gate is not None:
        g = _f64(out_gate)
        assert g.shape == out.shape
        out = out * g
    return out, sf
