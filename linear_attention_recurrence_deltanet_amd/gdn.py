"""ctypes binding of libgdn (C ABI in include/gdn.h).

Argument marshalling only: every step of the forward runs in the HIP kernels
of libgdn.so.  PyTorch supplies device memory and the current stream.  There
is no CPU fallback: if libgdn.so is missing or not built, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, -1, -2, -3
GDN_BF16, GDN_F32 = 0, 1

# every exported entry point of include/gdn.h
EXPORTS = ("gdn_default_opts", "gdn_fwd_chunked", "gdn_fwd_step", "gdn_fwd_step_noalloc", "gdn_fwd_bidir",
           "gdn_workspace_bytes", "gdn_bidir_workspace_bytes", "gdn_attn_sink_window",
           "gdn_attn_workspace_bytes", "gdn_fwd_framewise", "gdn_framewise_workspace_bytes",
           "gdn_strerror", "gdn_last_error", "gdn_version", "gdn_debug_flags")


class GdnOpts(ctypes.Structure):
    _fields_ = [("in_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int),
                ("qk_l2norm", ctypes.c_int),
                ("scale", ctypes.c_float),
                ("eps", ctypes.c_float),
                ("stream", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t),
                ("gate_logits", ctypes.c_int),
                ("out_gate", ctypes.c_void_p)]


class GdnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"libgdn status {status}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgdn.so not found at {path}: run "
                           "`python -m linear_attention_recurrence_deltanet_amd.build` first")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    fwd_args = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i]
    lib.gdn_fwd_chunked.argtypes = fwd_args + [i, ctypes.POINTER(GdnOpts)]
    lib.gdn_fwd_chunked.restype = i
    lib.gdn_fwd_step.argtypes = fwd_args + [ctypes.POINTER(GdnOpts)]
    lib.gdn_fwd_step.restype = i
    lib.gdn_fwd_step_noalloc.argtypes = fwd_args + [ctypes.POINTER(GdnOpts)]
    lib.gdn_fwd_step_noalloc.restype = i
    lib.gdn_fwd_bidir.argtypes = fwd_args + [i, ctypes.POINTER(GdnOpts)]
    lib.gdn_fwd_bidir.restype = i
    lib.gdn_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(GdnOpts)]
    lib.gdn_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_bidir_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(GdnOpts)]
    lib.gdn_bidir_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_attn_sink_window.argtypes = [vp, vp, vp, i, vp, vp, i, vp, vp, i, vp, i, i, i, i,
                                         ctypes.c_float, ctypes.POINTER(GdnOpts)]
    lib.gdn_attn_sink_window.restype = i
    lib.gdn_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(GdnOpts)]
    lib.gdn_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_fwd_framewise.argtypes = [vp] * 10 + [i] * 7 + [ctypes.POINTER(GdnOpts)]
    lib.gdn_fwd_framewise.restype = i
    lib.gdn_framewise_workspace_bytes.argtypes = [i] * 7 + [ctypes.POINTER(GdnOpts)]
    lib.gdn_framewise_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_default_opts.argtypes = [ctypes.POINTER(GdnOpts)]
    lib.gdn_default_opts.restype = None
    lib.gdn_strerror.argtypes = [i]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = i
    lib.gdn_debug_flags.argtypes = []
    lib.gdn_debug_flags.restype = i
    _lib = lib
    return lib


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_opts(in_dtype=torch.bfloat16, out_dtype=torch.float32, qk_l2norm=True, scale=1.0,
              eps=1e-6, stream=None, workspace: Optional[torch.Tensor] = None,
              gate_logits: bool = False, out_gate: Optional[torch.Tensor] = None) -> GdnOpts:
    o = GdnOpts()
    load().gdn_default_opts(ctypes.byref(o))
    o.in_dtype = _dtype_code(in_dtype)
    o.out_dtype = _dtype_code(out_dtype)
    o.qk_l2norm = 1 if qk_l2norm else 0
    o.scale = float(scale)
    o.eps = float(eps)
    if stream is None:
        stream = torch.cuda.current_stream()
    o.stream = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if workspace is not None:
        o.workspace = ctypes.c_void_p(workspace.data_ptr())
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    o.gate_logits = 1 if gate_logits else 0
    if out_gate is not None:
        o.out_gate = ctypes.c_void_p(out_gate.data_ptr())
    return o


def workspace_bytes(B, H, T, dk, dv, chunk=0, opts: Optional[GdnOpts] = None) -> int:
    return int(load().gdn_workspace_bytes(B, H, T, dk, dv, chunk,
                                          ctypes.byref(opts) if opts is not None else None))


def _workspace(workspace, B, H, T, dk, dv, chunk, in_dtype, out_dtype, device, bidir=False):
    """None: allocate what the plan needs; False: none (single-segment walk)."""
    if workspace is False:
        return None
    if workspace is not None:
        _check_workspace(workspace, device)
        return workspace
    o = GdnOpts()
    load().gdn_default_opts(ctypes.byref(o))
    o.in_dtype = _dtype_code(in_dtype)
    o.out_dtype = _dtype_code(out_dtype)
    query = load().gdn_bidir_workspace_bytes if bidir else load().gdn_workspace_bytes
    n = int(query(B, H, T, dk, dv, chunk, ctypes.byref(o)))
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def _check_workspace(ws, device):
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous device tensor on {device}")


def _on_stream(stream, *tensors):
    """Tensors this call allocated on the current stream but the kernels use on
    `stream`: tell the caching allocator, so their memory is not handed out
    again before the work on `stream` has finished."""
    if stream is None:
        return
    cur = torch.cuda.current_stream()
    sid = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if sid == cur.cuda_stream:
        return
    ext = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(sid)
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(ext)


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, load().gdn_last_error().decode())


def _prep(q, k, v, alpha, beta, state_in, out, state_out, out_dtype):
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v")
    if alpha.shape != (B, H, T) or beta.shape != (B, H, T):
        raise ValueError("alpha and beta must be [B, H, T]")
    _check_buf("state_in", state_in, (B, H, dk, dv), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, H, T, dv, dtype=out_dtype, device=q.device)
    else:
        _check_buf("out", out, (B, H, T, dv), (torch.float32, torch.bfloat16), q.device)
    if state_out is None:
        state_out = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device)
    else:
        _check_buf("state_out", state_out, (B, H, dk, dv), (torch.float32,), q.device)
    return B, H, T, dk, dv, out, state_out


def _check_buf(name, t, shape, dtypes, device):
    """A caller-supplied input or output buffer: the kernels see only its
    address, so its shape, dtype, device and layout are checked here."""
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")


def _check_gate(out_gate, q, B, H, T, dv):
    if out_gate is None:
        return
    if (not out_gate.is_cuda or out_gate.device != q.device or not out_gate.is_contiguous()
            or out_gate.dtype != q.dtype or tuple(out_gate.shape) != (B, H, T, dv)):
        raise ValueError("out_gate must be a contiguous device tensor [B, H, T, dv] of q's dtype")


def fwd_chunked(q, k, v, alpha, beta, state_in=None, chunk: int = 64, *, out=None, state_out=None,
                out_dtype=torch.float32, qk_l2norm=True, scale=1.0, eps=1e-6, stream=None,
                workspace=None, want_state: bool = True, gate_logits: bool = False, out_gate=None):
    """gdn_fwd_chunked.  Returns (out, state_out).

    workspace: None allocates the scratch the launch plan asks for (sequence
    split into segments when there are few heads); False passes none, which
    makes the library walk each sequence unsplit; or a uint8 device tensor.
    gate_logits: alpha and beta are logits (alpha = exp(-softplus(a)),
    beta = sigmoid(b) inside the kernel).  out_gate: multiplies out
    elementwise."""
    B, H, T, dk, dv, out, state_out = _prep(q, k, v, alpha, beta, state_in, out,
                                            state_out if want_state else None, out_dtype)
    if not want_state:
        state_out = None
    _check_gate(out_gate, q, B, H, T, dv)
    workspace = _workspace(workspace, B, H, T, dk, dv, chunk, q.dtype, out.dtype, q.device)
    opts = make_opts(q.dtype, out.dtype, qk_l2norm, scale, eps, stream, workspace, gate_logits, out_gate)
    _check(load().gdn_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(state_in), _ptr(out), _ptr(state_out),
                                  B, H, T, dk, dv, int(chunk), ctypes.byref(opts)))
    _on_stream(stream, workspace, out, state_out)
    return out, state_out


def fwd_step(q, k, v, alpha, beta, state_in=None, *, out=None, state_out=None,
             out_dtype=torch.float32, qk_l2norm=True, scale=1.0, eps=1e-6, stream=None,
             workspace=None, gate_logits: bool = False, out_gate=None):
    """gdn_fwd_step: one streaming chunk.  state_out may be state_in (in place).
    workspace, gate_logits and out_gate as for fwd_chunked."""
    B, H, T, dk, dv, out, state_out = _prep(q, k, v, alpha, beta, state_in, out, state_out,
                                            out_dtype)
    _check_gate(out_gate, q, B, H, T, dv)
    workspace = _workspace(workspace, B, H, T, dk, dv, 0, q.dtype, out.dtype, q.device)
    opts = make_opts(q.dtype, out.dtype, qk_l2norm, scale, eps, stream, workspace, gate_logits, out_gate)
    _check(load().gdn_fwd_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(state_in), _ptr(out), _ptr(state_out),
                               B, H, T, dk, dv, ctypes.byref(opts)))
    _on_stream(stream, workspace, out, state_out)
    return out, state_out


def fwd_step_noalloc(q, k, v, alpha, beta, state_in=None, *, out=None, state_out=None,
                     out_dtype=torch.float32, qk_l2norm=True, scale=1.0, eps=1e-6, stream=None,
                     gate_logits: bool = False, out_gate=None):
    """gdn_fwd_step_noalloc: gdn_fwd_step with its scratch in the library's
    static device array (the call allocates nothing on the device; outputs
    not given are allocated here, by torch, before the call)."""
    B, H, T, dk, dv, out, state_out = _prep(q, k, v, alpha, beta, state_in, out, state_out,
                                            out_dtype)
    _check_gate(out_gate, q, B, H, T, dv)
    opts = make_opts(q.dtype, out.dtype, qk_l2norm, scale, eps, stream, None, gate_logits, out_gate)
    _check(load().gdn_fwd_step_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(state_in), _ptr(out), _ptr(state_out),
                                       B, H, T, dk, dv, ctypes.byref(opts)))
    _on_stream(stream, out, state_out)
    return out, state_out


def fwd_bidir(q, k, v, alpha, beta, state_in=None, chunk: int = 0, *, out=None, state_out=None,
              out_dtype=torch.float32, qk_l2norm=True, scale=1.0, eps=1e-6, stream=None,
              workspace=None, gate_logits: bool = False, out_gate=None):
    """gdn_fwd_bidir: forward scan from state_in plus backward scan (zero state,
    reversed tokens) over one streaming chunk; out is the sum of the two
    scans' outputs and state_out the forward scan's final state.  chunk 0:
    the gdn_fwd_step tile.  workspace: None allocates gdn_bidir_workspace_bytes
    (bf16 outputs need it); other arguments as for fwd_chunked."""
    B, H, T, dk, dv, out, state_out = _prep(q, k, v, alpha, beta, state_in, out, state_out,
                                            out_dtype)
    _check_gate(out_gate, q, B, H, T, dv)
    workspace = _workspace(workspace, B, H, T, dk, dv, chunk, q.dtype, out.dtype, q.device,
                           bidir=True)
    opts = make_opts(q.dtype, out.dtype, qk_l2norm, scale, eps, stream, workspace, gate_logits, out_gate)
    _check(load().gdn_fwd_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(state_in), _ptr(out), _ptr(state_out),
                                B, H, T, dk, dv, int(chunk), ctypes.byref(opts)))
    _on_stream(stream, workspace, out, state_out)
    return out, state_out


def attn_sink_window(q, k_sink, v_sink, k_win, v_win, k_cur, v_cur, scale=None, *, out=None,
                     out_dtype=torch.float32, stream=None, workspace=None):
    """gdn_attn_sink_window: softmax(scale q K^T) V over [sink; window; current]
    keys.  q [B,H,Nq,d], k_x/v_x [B,H,n_x,d] bf16 device tensors (n_x may be
    0).  scale None: 1/sqrt(d).  workspace: None allocates what the split of
    the key range needs, False passes none (unsplit), or a uint8 device
    tensor.  Returns out [B,H,Nq,d]."""
    B, H, Nq, d = q.shape
    segs = []
    for name, k, v in (("sink", k_sink, v_sink), ("win", k_win, v_win), ("cur", k_cur, v_cur)):
        for t in (k, v):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
                raise ValueError(f"{name} keys and values must be contiguous bf16 device tensors")
        if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d:
            raise ValueError(f"{name} keys and values must be [B, H, n, d]")
        segs.append((k, v, k.shape[2]))
    if not q.is_cuda or not q.is_contiguous() or q.dtype != torch.bfloat16:
        raise ValueError("q must be a contiguous bf16 device tensor")
    for name, k, v in (("sink", k_sink, v_sink), ("win", k_win, v_win), ("cur", k_cur, v_cur)):
        if k.device != q.device or v.device != q.device:
            raise ValueError(f"{name} keys and values must be on {q.device}")
    if out is None:
        out = torch.empty(B, H, Nq, d, dtype=out_dtype, device=q.device)
    else:
        _check_buf("out", out, (B, H, Nq, d), (torch.float32, torch.bfloat16), q.device)
    if workspace is not None and workspace is not False:
        _check_workspace(workspace, q.device)
    if workspace is None:
        n = int(load().gdn_attn_workspace_bytes(B, H, Nq, k_sink.shape[2], k_win.shape[2],
                                                k_cur.shape[2], d, None))
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    elif workspace is False:
        workspace = None
    opts = make_opts(q.dtype, out.dtype, stream=stream, workspace=workspace)
    args = []
    for k, v, n in segs:
        args += [_ptr(k) if n else None, _ptr(v) if n else None, int(n)]
    _check(load().gdn_attn_sink_window(_ptr(q), *args, _ptr(out), B, H, Nq, d,
                                       float(scale) if scale else 0.0, ctypes.byref(opts)))
    _on_stream(stream, workspace, out)
    return out


def framewise_workspace_bytes(B, H, F, N, dk, dv) -> int:
    return int(load().gdn_framewise_workspace_bytes(B, H, F, N, dk, dv, 0, None))


def fwd_framewise(q, k, v, alpha, beta, frame_len: int, state_in=None, z_in=None, *,
                  out=None, state_out=None, z_out=None, out_dtype=torch.float32, qk_l2norm=True,
                  eps=1e-6, stream=None, workspace=None, gate_logits: bool = False, out_gate=None):
    """gdn_fwd_framewise: frame-wise gated delta rule with a normalised
    readout over F = T / frame_len frames (one state update per frame).
    q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T] and alpha [B,H,F] bf16
    device tensors; state_in [B,H,dk,dv] and z_in [B,H,dk] fp32 or None.
    workspace: None allocates gdn_framewise_workspace_bytes, or a uint8
    device tensor.  Returns (out, state_out, z_out); state_out may be
    state_in and z_out z_in (in place)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor on q's device")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = int(frame_len)
    if N <= 0 or T % N:
        raise ValueError("T must be a whole number of frames")
    F = T // N
    if k.shape != q.shape or v.shape[:3] != (B, H, T) or beta.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, beta")
    if alpha.shape != (B, H, F):
        raise ValueError("alpha must be [B, H, F]")
    _check_buf("state_in", state_in, (B, H, dk, dv), (torch.float32,), q.device)
    _check_buf("z_in", z_in, (B, H, dk), (torch.float32,), q.device)
    _check_gate(out_gate, q, B, H, T, dv)
    if out is None:
        out = torch.empty(B, H, T, dv, dtype=out_dtype, device=q.device)
    else:
        _check_buf("out", out, (B, H, T, dv), (torch.float32, torch.bfloat16), q.device)
    if state_out is None:
        state_out = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device)
    else:
        _check_buf("state_out", state_out, (B, H, dk, dv), (torch.float32,), q.device)
    if z_out is None:
        z_out = torch.empty(B, H, dk, dtype=torch.float32, device=q.device)
    else:
        _check_buf("z_out", z_out, (B, H, dk), (torch.float32,), q.device)
    if workspace is None:
        n = framewise_workspace_bytes(B, H, F, N, dk, dv)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    opts = make_opts(q.dtype, out.dtype, qk_l2norm, 1.0, eps, stream, workspace, gate_logits, out_gate)
    _check(load().gdn_fwd_framewise(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(state_in), _ptr(z_in), _ptr(out), _ptr(state_out), _ptr(z_out),
                                    B, H, F, N, dk, dv, 0, ctypes.byref(opts)))
    _on_stream(stream, workspace, out, state_out, z_out)
    return out, state_out, z_out
