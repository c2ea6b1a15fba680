"""Seeded synthetic inputs for the Gated DeltaNet forward.

This module holds only random draws and the workload table: no step of the
method's arithmetic.  Both the GPU tests/benchmark and the fp64 oracle take
their inputs from here, so they read exactly the same bits.

Input recipe, per head and token (SANA-Streaming, paperpeel page, section 2.1:
per-head q, k, v with a decay gate alpha and a write gate beta; section 4.1:
1280x704 video through a 32x32 VAE gives 40x22 = 880 tokens per latent frame,
and a streaming chunk holds 3 latent frames = 2640 tokens):

  q, k ~ N(0, 1), each token rescaled to unit L2 norm in fp32;
  v    ~ N(0, 1);
  alpha = exp(-softplus(N(mu_a, sigma_a)))      (decay, in (0, 1))
  beta  = sigmoid(N(mu_b, sigma_b))             (write strength, in (0, 1))
  state = N(0, sigma_s) in fp32, or zero;
then cast to the workload's input dtype.  N(mu, sigma) means mean and
standard deviation.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int              # tokens per call
    dk: int
    dv: int
    chunk: int          # kernel tile length in tokens
    dtype: str          # "bf16" or "f32" for q, k, v, alpha, beta
    calls: int          # successive calls with the state carried
    alpha_mu: float
    alpha_sigma: float
    beta_mu: float
    beta_sigma: float
    state_sigma: Optional[float]   # None: zero initial state
    seed: int

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, named by what they are.
WORKLOADS = {
    # one head, fp32 inputs, correctness only
    "tiny_f32": Workload("tiny_f32", 1, 1, 256, 32, 32, 64, "f32", 1,
                         0.0, 1.0, 0.0, 1.0, None, 1000),
    # one streaming chunk (3 latent frames x 880 tokens), 16 heads of 64
    "stream_chunk_h16_d64": Workload("stream_chunk_h16_d64", 1, 16, 2640, 64, 64, 64, "bf16", 1,
                                     -3.0, 1.0, 0.0, 1.0, 0.02, 1001),
    # 20 successive streaming chunks, 16 heads of 128, state carried
    "rollout_h16_d128": Workload("rollout_h16_d128", 1, 16, 2640, 128, 128, 64, "bf16", 20,
                                 0.0, 1.0, 0.0, 1.0, None, 1002),
    # batched long prefill, 4 x 32 heads of 128, 16384 tokens
    "prefill_b4_h32_d128": Workload("prefill_b4_h32_d128", 4, 32, 16384, 128, 128, 64, "bf16", 1,
                                    0.0, 1.0, 0.0, 1.0, None, 1003),
    # 200 successive single-frame calls (880 tokens), 2 x 24 heads of 128
    "frame_step_b2_h24_d128": Workload("frame_step_b2_h24_d128", 2, 24, 880, 128, 128, 64, "bf16", 200,
                                       -5.0, 0.5, 1.0, 1.0, None, 1004),
}


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # recipe step: each token vector rescaled to unit length (fp32)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def make_call(wl: Workload, call: int = 0, *, B: Optional[int] = None, H: Optional[int] = None,
              T: Optional[int] = None, gates: bool = False):
    """Draw the inputs of call number `call` (CPU tensors in the workload dtype).

    B, H, T may be overridden (smaller tests) while keeping the distribution.
    Returns dict(q, k, v, alpha, beta) plus 'state_in' (fp32, or None).
    gates: also 'alpha_logit', 'beta_logit' (the normal draws alpha and beta
    are mapped from, in the workload dtype) and 'out_gate' ([B,H,T,dv],
    sigmoid of a standard normal draw), drawn after everything else so that
    the other inputs do not change.
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed * 100003 + call)
    f32 = torch.float32
    q = _unit_rows(torch.randn(B, H, T, wl.dk, generator=g, dtype=f32))
    k = _unit_rows(torch.randn(B, H, T, wl.dk, generator=g, dtype=f32))
    v = torch.randn(B, H, T, wl.dv, generator=g, dtype=f32)
    za = torch.randn(B, H, T, generator=g, dtype=f32) * wl.alpha_sigma + wl.alpha_mu
    zb = torch.randn(B, H, T, generator=g, dtype=f32) * wl.beta_sigma + wl.beta_mu
    alpha = torch.exp(-torch.nn.functional.softplus(za))
    beta = torch.sigmoid(zb)
    state = None
    if call == 0 and wl.state_sigma is not None:
        state = torch.randn(B, H, wl.dk, wl.dv, generator=g, dtype=f32) * wl.state_sigma
    dt = wl.torch_dtype
    d = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), alpha=alpha.to(dt), beta=beta.to(dt),
             state_in=state)
    if gates:
        d["alpha_logit"] = za.to(dt)
        d["beta_logit"] = zb.to(dt)
        d["out_gate"] = torch.sigmoid(torch.randn(B, H, T, wl.dv, generator=g, dtype=f32)).to(dt)
    return d


def to_numpy64(t: torch.Tensor):
    """Exact upcast of a CPU tensor (bf16/fp32) to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


# ---------------------------------------------------------------------------
# Softmax attention with a persistent sink and a recent window (the other block
# type of the hybrid: SANA-Streaming section 2.1, "Softmax blocks for local
# window and sink refinement"): the current streaming chunk attends, with no
# mask, to the sink chunk (the stream's first chunk), a window of recent
# chunks and itself.  q, k, v ~ N(0, 1) in bf16; lengths in tokens.

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    Nq: int             # query tokens (the current chunk)
    n_sink: int         # tokens of the sink chunk
    n_win: int          # tokens of the recent window
    n_cur: int          # tokens of the current chunk (keys and values)
    d: int              # head dimension
    seed: int

    def replace(self, **kw) -> "AttnWorkload":
        return dataclasses.replace(self, **kw)


ATTN_WORKLOADS = {
    # one streaming chunk (3 latent frames, 2640 tokens) attending to a sink
    # chunk, one recent chunk and itself: 16 heads of 64
    "attn_chunk_h16_d64": AttnWorkload("attn_chunk_h16_d64", 1, 16, 2640, 2640, 2640, 2640, 64, 2001),
    # the same with 8 heads of 128
    "attn_chunk_h8_d128": AttnWorkload("attn_chunk_h8_d128", 1, 8, 2640, 2640, 2640, 2640, 128, 2002),
}


def make_attn_call(wl: AttnWorkload, call: int = 0, *, B: Optional[int] = None, H: Optional[int] = None,
                   Nq: Optional[int] = None, n_sink: Optional[int] = None, n_win: Optional[int] = None,
                   n_cur: Optional[int] = None):
    """q [B,H,Nq,d] and k_x, v_x [B,H,n_x,d] for x in sink, win, cur (bf16 CPU
    tensors, standard normal draws); sizes may be overridden."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    Nq = wl.Nq if Nq is None else Nq
    ns = wl.n_sink if n_sink is None else n_sink
    nw = wl.n_win if n_win is None else n_win
    nc = wl.n_cur if n_cur is None else n_cur
    g = torch.Generator().manual_seed(wl.seed * 1000 + call)
    bf = torch.bfloat16
    r = lambda n: torch.randn(B, H, n, wl.d, generator=g, dtype=torch.float32).to(bf)
    d = dict(q=r(Nq))
    for name, n in (("sink", ns), ("win", nw), ("cur", nc)):
        d["k_" + name] = r(n)
        d["v_" + name] = r(n)
    return d



# ---------------------------------------------------------------------------
# Frame-wise Gated DeltaNet with a normalised readout (SANA-Streaming section
# 2.1, "Frame-wise Gated DeltaNet"): a call holds F latent frames of N tokens;
# one decay per frame, one write strength per token, an output gate per
# element.  The readout divides by z . q, so the features must keep that
# denominator away from zero: q and k are drawn non-negative (absolute values
# of standard normal draws, then unit rows in fp32), as feature maps of
# normalised linear attention are; with sign-symmetric draws z . q takes
# either sign.
#
#   q, k = unit rows of |N(0, 1)|;  v ~ N(0, 1)
#   alpha [F]   = exp(-softplus(N(mu_a, sigma_a)))
#   beta  [F*N] = sigmoid(N(mu_b, sigma_b))
#   out_gate    = sigmoid(N(0, 1))
#   zero numerator and denominator states before the first call.

@dataclasses.dataclass(frozen=True)
class FrameWorkload:
    name: str
    B: int
    H: int
    F: int              # frames per call
    N: int              # tokens per frame
    dk: int
    dv: int
    calls: int          # successive calls with both states carried
    alpha_mu: float
    alpha_sigma: float
    beta_mu: float
    beta_sigma: float
    seed: int

    @property
    def T(self) -> int:
        return self.F * self.N

    def replace(self, **kw) -> "FrameWorkload":
        return dataclasses.replace(self, **kw)


FRAME_WORKLOADS = {
    # one streaming chunk of 3 latent frames x 880 tokens, 16 heads of 64
    "frame_stream_h16_d64": FrameWorkload("frame_stream_h16_d64", 1, 16, 3, 880, 64, 64, 1,
                                          0.0, 1.0, 0.0, 1.0, 3001),
    # 20 successive streaming chunks, 16 heads of 128, both states carried
    "frame_rollout_h16_d128": FrameWorkload("frame_rollout_h16_d128", 1, 16, 3, 880, 128, 128, 20,
                                            0.0, 1.0, 0.0, 1.0, 3002),
}


def make_frame_call(wl: FrameWorkload, call: int = 0, *, B: Optional[int] = None,
                    H: Optional[int] = None, F: Optional[int] = None, N: Optional[int] = None):
    """Inputs of call number `call` (bf16 CPU tensors): q, k [B,H,F*N,dk],
    v and out_gate [B,H,F*N,dv], alpha [B,H,F], beta [B,H,F*N], and
    'alpha_logit', 'beta_logit': the normal draws alpha and beta are mapped
    from.  Sizes may be overridden."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    F = wl.F if F is None else F
    N = wl.N if N is None else N
    T = F * N
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed * 100003 + call)
    f32, bf = torch.float32, torch.bfloat16
    q = _unit_rows(torch.randn(B, H, T, wl.dk, generator=g, dtype=f32).abs())
    k = _unit_rows(torch.randn(B, H, T, wl.dk, generator=g, dtype=f32).abs())
    v = torch.randn(B, H, T, wl.dv, generator=g, dtype=f32)
    za = torch.randn(B, H, F, generator=g, dtype=f32) * wl.alpha_sigma + wl.alpha_mu
    zb = torch.randn(B, H, T, generator=g, dtype=f32) * wl.beta_sigma + wl.beta_mu
    og = torch.sigmoid(torch.randn(B, H, T, wl.dv, generator=g, dtype=f32))
    return dict(q=q.to(bf), k=k.to(bf), v=v.to(bf),
                alpha=torch.exp(-torch.nn.functional.softplus(za)).to(bf),
                beta=torch.sigmoid(zb).to(bf), out_gate=og.to(bf),
                alpha_logit=za.to(bf), beta_logit=zb.to(bf))
