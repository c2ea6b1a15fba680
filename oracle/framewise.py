"""fp64 oracle of frame-wise Gated DeltaNet with a normalised readout --
TEST INFRASTRUCTURE ONLY (imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the GPU library).

Source: SANA-Streaming (paperpeel page), section 2.1 "Frame-wise Gated
DeltaNet for Global Accumulated Memory": per head, latents of F frames of N
tokens give q, k, v, a decay gate alpha in R^F (one per frame), a write gate
beta in R^{F x N} (one per token) and an output gate g in R^{F x N x C}; a
numerator state S^kv and a denominator (normaliser) state S^z are updated
with the delta-rule correction and carried across chunks.  Appendix G.3 names
the same three gates; G.4 ("Frame-wise delta-rule update") and G.5
("Normalized readout") survive as headings only, so the update and readout
equations are readings:

  * within a frame the tokens are written one after another by the
    token-wise delta rule, and the frame's decay alpha_f multiplies both
    states once, before the frame's first token is written;
  * the denominator state z (a d_k vector) follows the same recurrence as
    every column of the numerator state, with a value of constant 1;
  * the output of token t is (S_t q_t) / (z_t . q_t), then multiplied
    elementwise by the output gate.

Plain token loop, vectorised over (batch, head) only; no chunking.

Pins (tests/test_oracle_pins.py): equality with the C token-wise oracle run
with the frame decays placed on each frame's first token (numerator) and on a
value column of ones (denominator); closed forms for beta = 0, constant
values, shifted values, orthonormal keys; split invariance across calls.  The
readings above have no printed values on the pages to pin them against.
"""
from __future__ import annotations

import numpy as np

DEFAULT_EPS = 1e-6


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def gdn_framewise(q, k, v, alpha, beta, frame_len, state_in=None, z_in=None, *, out_gate=None,
                  qk_l2norm=True, eps=DEFAULT_EPS):
    """Frame-wise gated delta rule with a normalised readout, fp64.

    Shapes: q, k [B,H,T,dk], v [B,H,T,dv] with T = F * frame_len; alpha
    [B,H,F] (one decay per frame); beta [B,H,T]; state_in [B,H,dk,dv] (the
    transposed numerator state M = S^T) or None; z_in [B,H,dk] or None (zero
    states); out_gate [B,H,T,dv] or None.
    Returns (out [B,H,T,dv], state_out [B,H,dk,dv], z_out [B,H,dk]).
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = int(frame_len)
    assert N >= 1 and T % N == 0, "a call holds whole frames"
    F = T // N
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, F) and beta.shape == (B, H, T)
    M = np.zeros((B, H, dk, dv)) if state_in is None else _f64(state_in).copy()
    z = np.zeros((B, H, dk)) if z_in is None else _f64(z_in).copy()
    assert M.shape == (B, H, dk, dv) and z.shape == (B, H, dk)
    if qk_l2norm:
        q = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
        k = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    out = np.empty((B, H, T, dv))
    for f in range(F):
        a = alpha[:, :, f]
        M *= a[:, :, None, None]          # the frame's decay, once
        z *= a[:, :, None]
        for n in range(N):
            t = f * N + n
            kt, qt, b = k[:, :, t], q[:, :, t], beta[:, :, t]
            # delta-rule correction: the write replaces beta of what the state
            # recalls for k_t by beta of the new value (1 for the normaliser)
            recall = np.einsum("bhi,bhij->bhj", kt, M)
            M += np.einsum("bhi,bhj->bhij", kt, b[:, :, None] * (v[:, :, t] - recall))
            z += kt * (b * (1.0 - np.einsum("bhi,bhi->bh", kt, z)))[:, :, None]
            num = np.einsum("bhij,bhi->bhj", M, qt)
            den = np.einsum("bhi,bhi->bh", z, qt)
            out[:, :, t] = num / den[:, :, None]
    if out_gate is not None:
        g = _f64(out_gate)
        assert g.shape == out.shape
        out = out * g
    return out, M, z
