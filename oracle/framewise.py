"""fp64 oracle of frame-wise Gated DeltaNet with a normalised readout --
TEST INFRASTRUCTURE ONLY (imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the GPU library).

Source: SANA-Streaming (paperpeel page), section 2.1 "Frame-wise Gated
DeltaNet for Global Accumulated Memory": per head, latents of F frames of N
tokens give q, k, v, a decay gate alpha in R^F (one per frame), a write gate
beta in R^{F x N} (one per token) and an output gate g in R^{F x N x C}; the
state is updated frame by frame rather than token by token, with the
delta-rule correction, as a numerator state S^kv and a denominator
(normaliser) state S^z carried across chunks.  Section 2.3 "Efficient GDN
Kernel" computes it in three phases: frame summaries by reductions over the
spatial tokens, a short recurrent scan over frames, and the frame's queries
read against the frame's state.  Appendix G.4 ("Frame-wise delta-rule
update") and G.5 ("Normalized readout") survive as headings only, so the
equations are readings:

  * one update per frame, from the frame's mean over its N tokens (the
    delta rule is one gradient step on ||S k - v||^2 / 2 with step beta; the
    frame-wise update is one step on the frame's mean loss
    (1/N) sum_n beta_n ||S k_n - v_n||^2 / 2, taken from the decayed state):
        G_f = (1/N) sum_n beta_{f,n} k_n k_n^T
        S_f = alpha_f S_{f-1} (I - G_f) + (1/N) sum_n beta_{f,n} v_n k_n^T
    With beta in [0, 1] and unit keys, I - G_f has eigenvalues in [0, 1], so
    the state stays bounded however many tokens a frame holds; at N = 1 it is
    the token-wise gated delta rule;
  * the denominator z (a d_k row vector) follows the same update with a
    value of constant 1: z_f = alpha_f z_{f-1} (I - G_f) + (1/N) sum_n beta k_n^T;
  * every token of frame f reads the frame's updated state:
        out_{f,n} = (S_f q_n) / (z_f . q_n), then times the output gate.

Plain loop over frames, vectorised over (batch, head); sums over the frame's
tokens written out with einsum.  The state is stored transposed, M = S^T
[d_k][d_v], as in the token-wise oracle.

Pins (tests/test_oracle_pins.py): N = 1 equals the C token-wise oracle;
keys orthonormal within each frame equal the token-wise scan with beta / N at
frame ends; beta = 0 decays only; one autograd gradient step on the frame's
mean loss; permutation of a frame's tokens; N equal tokens equal one token;
constant values read back; shifted values; split invariance across calls.
The readings themselves have no printed values on the pages to pin them
against.
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
        sl = slice(f * N, (f + 1) * N)
        kf, vf, qf, bf = k[:, :, sl], v[:, :, sl], q[:, :, sl], beta[:, :, sl]
        a = alpha[:, :, f]
        # frame summaries: the means over the frame's tokens
        G = np.einsum("bhn,bhni,bhnj->bhij", bf, kf, kf) / N
        Wv = np.einsum("bhn,bhni,bhnj->bhij", bf, kf, vf) / N
        Wz = np.einsum("bhn,bhni->bhi", bf, kf) / N
        # one decayed delta-rule step per frame: M <- alpha (I - G) M + Wv
        M = a[:, :, None, None] * (M - np.einsum("bhik,bhkj->bhij", G, M)) + Wv
        z = a[:, :, None] * (z - np.einsum("bhik,bhk->bhi", G, z)) + Wz
        # every token of the frame reads the frame's updated state
        num = np.einsum("bhij,bhni->bhnj", M, qf)
        den = np.einsum("bhi,bhni->bhn", z, qf)
        out[:, :, sl] = num / den[..., None]
    if out_gate is not None:
        g = _f64(out_gate)
        assert g.shape == out.shape
        out = out * g
    return out, M, z
