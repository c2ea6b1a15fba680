"""fp64 CPU oracle of the sink-and-window softmax attention block -- TEST
INFRASTRUCTURE ONLY (tests/, the smoke check and bench.py's cpu_baseline leg
may import it; the GPU library never does, and they share no code).

What it computes (SANA-Streaming, paperpeel page, section 2.1 "Softmax blocks
for local window and sink refinement": instead of all previous frames, each
chunk attends to a constrained context made of itself, a persistent sink
chunk shared across the stream, and a short window of recent chunks; sinks
after Xiao et al. [30]):

    per (b, h):  K = [K_sink; K_win; K_cur],  V = [V_sink; V_win; V_cur]
                 S = scale * Q K^T             (Nq x N, N = n_sink + n_win + n_cur)
                 P = softmax(S) along the keys  (row max subtracted first)
                 O = P V

No mask: every query of the chunk sees every key of the context (the video
model denoises a whole chunk at once).  scale None means 1 / sqrt(d).
Parity pins: tests/test_oracle_pins.py (closed forms, the log-sum-exp split
identity, key permutation, and an independent library attention in fp64).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def attn_sink_window(q, k_sink, v_sink, k_win, v_win, k_cur, v_cur, scale=None):
    """q [B,H,Nq,d]; k_x, v_x [B,H,n_x,d] (n_x may be 0).  Returns O [B,H,Nq,d] fp64."""
    q = _f64(q)
    K = np.concatenate([_f64(k_sink), _f64(k_win), _f64(k_cur)], axis=2)
    V = np.concatenate([_f64(v_sink), _f64(v_win), _f64(v_cur)], axis=2)
    B, H, Nq, d = q.shape
    assert K.shape[:2] == (B, H) and K.shape[3] == d and V.shape == K.shape
    assert K.shape[2] > 0, "empty context"
    s = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.empty((B, H, Nq, d))
    for b in range(B):
        for h in range(H):
            S = s * (q[b, h] @ K[b, h].T)
            S -= S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[b, h] = P @ V[b, h]
    return out
