"""Pins of the fp64 oracle against facts fixed by the mathematics of the
gated delta rule (SANA-Streaming section 2.1; Gated DeltaNet [35]), not by the
oracle itself: hand-worked golden examples, closed forms of special cases, an
explicitly unrolled product of d_k x d_k matrices, per-step identities,
contraction and split invariance.  Each test targets a plausible mistake
(dropped term, wrong sign, wrong index, transposed operand, missing
normalisation).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(rng, B=1, H=1, T=20, dk=6, dv=5, state=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    a = np.exp(-np.log1p(np.exp(rng.standard_normal((B, H, T)))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    s = rng.standard_normal((B, H, dk, dv)) * 0.5 if state else None
    return q, k, v, a, b, s


# ----------------------------------------------------------------- golden


@pytest.mark.parametrize("name", ["worked_example_1.json", "worked_example_2.json"])
def test_golden_worked_examples(oracle_mod, name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    F = lambda a: np.array([[float(Fraction(x)) for x in row] for row in a])
    q, k, v = F(g["q"]), F(g["k"]), F(g["v"])
    a = np.array([float(Fraction(x)) for x in g["alpha"]])
    b = np.array([float(Fraction(x)) for x in g["beta"]])
    s = None if g["state_in"] is None else F(g["state_in"])[None, None]
    out, st = oracle_mod.gdn_fwd(q[None, None], k[None, None], v[None, None], a[None, None],
                                 b[None, None], s, eps=0.0)
    np.testing.assert_allclose(out[0, 0], F(g["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st[0, 0], F(g["state_out"]), rtol=0, atol=1e-14)


# ------------------------------------------------------------ closed forms


def test_beta_zero_pure_decay(oracle_mod):
    """beta = 0: no write and no erase, so M_t = gamma_t M_0, o_t = gamma_t M_0^T q_t."""
    rng = np.random.default_rng(1)
    q, k, v, a, _, s = rand_case(rng, T=30)
    b = np.zeros_like(a)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    gam = np.cumprod(a[0, 0])
    qh = unit(q[0, 0])
    ref = gam[:, None] * (qh @ s[0, 0])
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st[0, 0], gam[-1] * s[0, 0], rtol=1e-12, atol=1e-13)
    # alpha = 1 as well: the state is unchanged
    out1, st1 = oracle_mod.gdn_fwd(q, k, v, np.ones_like(a), b, s, eps=0.0)
    np.testing.assert_allclose(st1[0, 0], s[0, 0], rtol=0, atol=1e-14)


def test_small_beta_is_causal_linear_attention(oracle_mod):
    """alpha = 1, M0 = 0, beta = eps*b: o_t / eps -> sum_{s<=t} b_s (k_s . q_t) v_s."""
    rng = np.random.default_rng(2)
    q, k, v, _, bb, _ = rand_case(rng, T=25, dk=8, dv=4, state=False)
    a = np.ones_like(bb)
    eps = 1e-7
    out, _ = oracle_mod.gdn_fwd(q, k, v, a, eps * bb, None, eps=0.0)
    qh, kh = unit(q[0, 0]), unit(k[0, 0])
    scores = np.tril(qh @ kh.T) * bb[0, 0][None, :]
    ref = scores @ v[0, 0]
    np.testing.assert_allclose(out[0, 0] / eps, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_orthonormal_keys_gated_linear_attention(oracle_mod):
    """Orthonormal keys decouple the delta correction: for M0 = 0,
    o_t = sum_{s<=t} exp(g_t - g_s) beta_s (k_s . q_t) v_s exactly."""
    rng = np.random.default_rng(3)
    T, dk, dv = 12, 16, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None] * rng.uniform(0.5, 2.0, size=(1, 1, T, 1))   # normalised inside
    q = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    a = rng.uniform(0.3, 1.0, size=(1, 1, T))
    b = rng.uniform(0.0, 1.0, size=(1, 1, T))
    out, _ = oracle_mod.gdn_fwd(q, k, v, a, b, None, eps=0.0)
    g = np.cumsum(np.log(a[0, 0]))
    G = np.tril(np.exp(g[:, None] - g[None, :]))
    ref = (G * (unit(q[0, 0]) @ Qm[:T].T) * b[0, 0][None, :]) @ v[0, 0]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_exact_retrieval(oracle_mod):
    """beta = alpha = 1, orthonormal keys: querying with an earlier key
    returns exactly the value written with it."""
    rng = np.random.default_rng(4)
    T, dk, dv = 10, 10, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None]
    pick = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = Qm[pick][None, None]
    v = rng.standard_normal((1, 1, T, dv))
    one = np.ones((1, 1, T))
    out, _ = oracle_mod.gdn_fwd(q, k, v, one, one, None, eps=0.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0][pick], rtol=0, atol=1e-12)


def test_identical_keys_projector(oracle_mod):
    """k_t = k for all t, alpha = beta = 1: M_t = (I - k k^T) M0 + k v_t^T, so
    o_t = (q.k) v_t + q^T (I - k k^T) M0 (worst-case collinear keys)."""
    rng = np.random.default_rng(5)
    T, dk, dv = 15, 6, 4
    kk = unit(rng.standard_normal(dk))
    k = np.tile(kk, (1, 1, T, 1)) * 3.0
    q = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    s = rng.standard_normal((1, 1, dk, dv))
    one = np.ones((1, 1, T))
    out, st = oracle_mod.gdn_fwd(q, k, v, one, one, s, eps=0.0)
    Pm = np.eye(dk) - np.outer(kk, kk)
    qh = unit(q[0, 0])
    ref = (qh @ kk)[:, None] * v[0, 0] + qh @ Pm @ s[0, 0]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], Pm @ s[0, 0] + np.outer(kk, v[0, 0, -1]), atol=1e-12)


def test_dk_one_is_ema(oracle_mod):
    """dk = 1: k^ = sign(k); m_t = alpha_t (1 - beta_t) m_{t-1} + beta_t sign(k_t) v_t."""
    rng = np.random.default_rng(6)
    T, dv = 40, 3
    q, k, v, a, b, s = rand_case(rng, T=T, dk=1, dv=dv)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    m = s[0, 0, 0].copy()
    for t in range(T):
        sk = np.sign(k[0, 0, t, 0])
        # the erase term uses k^2 = 1 and the write term k^ v
        m = a[0, 0, t] * (1 - b[0, 0, t]) * m + b[0, 0, t] * sk * v[0, 0, t]
        np.testing.assert_allclose(out[0, 0, t], np.sign(q[0, 0, t, 0]) * m, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0, 0, 0], m, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- independent forms


def test_unrolled_matrix_product(oracle_mod):
    """M_T = P_T..P_1 M0 + sum_t P_T..P_{t+1} beta_t k_t v_t^T with
    P_t = alpha_t (I - beta_t k_t k_t^T) as dense dk x dk matrices, and every
    o_t = M_t^T q_t; S form S_t = alpha S (I - beta k k^T) + beta v k^T too."""
    rng = np.random.default_rng(7)
    T, dk, dv = 24, 7, 5
    q, k, v, a, b, s = rand_case(rng, T=T, dk=dk, dv=dv)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    qh, kh = unit(q[0, 0]), unit(k[0, 0])
    Ps = [a[0, 0, t] * (np.eye(dk) - b[0, 0, t] * np.outer(kh[t], kh[t])) for t in range(T)]
    for t in range(T):
        # product P_t ... P_0 applied to M0, plus the writes
        prod = np.eye(dk)
        for j in range(t + 1):
            prod = Ps[j] @ prod
        Mt = prod @ s[0, 0]
        for u in range(t + 1):
            tail = np.eye(dk)
            for j in range(u + 1, t + 1):
                tail = Ps[j] @ tail
            Mt = Mt + tail @ (b[0, 0, u] * np.outer(kh[u], v[0, 0, u]))
        np.testing.assert_allclose(out[0, 0, t], Mt.T @ qh[t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], Mt, rtol=1e-11, atol=1e-12)
    # S form, written directly from the recurrence
    S = s[0, 0].T.copy()
    for t in range(T):
        S = a[0, 0, t] * S @ (np.eye(dk) - b[0, 0, t] * np.outer(kh[t], kh[t])) \
            + b[0, 0, t] * np.outer(v[0, 0, t], kh[t])
        np.testing.assert_allclose(out[0, 0, t], S @ qh[t], rtol=1e-11, atol=1e-12)


def test_per_step_identity_and_contraction(oracle_mod):
    """For unit k: S_t k_t = alpha_t (1 - beta_t) S_{t-1} k_t + beta_t v_t
    (beta = 1 stores v_t exactly along k_t), and ||S_t|| <= alpha_t ||S_{t-1}|| + beta_t ||v_t||."""
    rng = np.random.default_rng(8)
    T, dk, dv = 30, 8, 6
    q, k, v, a, b, s = rand_case(rng, T=T, dk=dk, dv=dv)
    b[0, 0, ::5] = 1.0
    M = s.copy()
    for t in range(T):
        sl = slice(t, t + 1)
        _, M1 = oracle_mod.gdn_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl], b[:, :, sl], M, eps=0.0)
        kh = unit(k[0, 0, t])
        lhs = M1[0, 0].T @ kh
        rhs = a[0, 0, t] * (1 - b[0, 0, t]) * (M[0, 0].T @ kh) + b[0, 0, t] * v[0, 0, t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        n0, n1 = np.linalg.norm(M[0, 0], 2), np.linalg.norm(M1[0, 0], 2)
        assert n1 <= a[0, 0, t] * n0 + b[0, 0, t] * np.linalg.norm(v[0, 0, t]) + 1e-12
        M = M1


def test_split_invariance(oracle_mod):
    """Running [0, t1) then [t1, T) with the state carried equals one run."""
    rng = np.random.default_rng(9)
    q, k, v, a, b, s = rand_case(rng, B=2, H=3, T=50, dk=8, dv=12)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    for t1 in (1, 17, 49):
        o1, s1 = oracle_mod.gdn_fwd(q[:, :, :t1], k[:, :, :t1], v[:, :, :t1], a[:, :, :t1], b[:, :, :t1], s, eps=0.0)
        o2, s2 = oracle_mod.gdn_fwd(q[:, :, t1:], k[:, :, t1:], v[:, :, t1:], a[:, :, t1:], b[:, :, t1:], s1, eps=0.0)
        np.testing.assert_allclose(np.concatenate([o1, o2], 2), out, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s2, st, rtol=1e-13, atol=1e-13)


def test_heads_are_independent_and_ordered(oracle_mod):
    """Each (b, h) runs alone; catches mixed-up head strides."""
    rng = np.random.default_rng(10)
    q, k, v, a, b, s = rand_case(rng, B=2, H=3, T=9, dk=4, dv=20)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    for bi in range(2):
        for hi in range(3):
            sl = (slice(bi, bi + 1), slice(hi, hi + 1))
            o1, s1 = oracle_mod.gdn_fwd(q[sl], k[sl], v[sl], a[sl], b[sl], s[sl], eps=0.0)
            np.testing.assert_array_equal(o1[0, 0], out[bi, hi])
            np.testing.assert_array_equal(s1[0, 0], st[bi, hi])


def test_normalisation_scale_and_eps(oracle_mod):
    """qk_l2norm = 0 uses q, k as given; scale multiplies q^; eps enters the
    norm as sqrt(|x|^2 + eps)."""
    rng = np.random.default_rng(11)
    q, k, v, a, b, s = rand_case(rng, T=6, dk=3, dv=2)
    qn, kn = unit(q), unit(k)
    o_pre, s_pre = oracle_mod.gdn_fwd(qn, kn, v, a, b, s, qk_l2norm=False, scale=1.0, eps=0.0)
    o_in, s_in = oracle_mod.gdn_fwd(q, k, v, a, b, s, qk_l2norm=True, eps=0.0)
    np.testing.assert_allclose(o_in, o_pre, rtol=1e-12, atol=1e-13)
    o_sc, _ = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0, scale=0.125)
    np.testing.assert_allclose(o_sc, 0.125 * o_in, rtol=1e-12, atol=1e-14)
    # a tiny key: eps dominates, k^ ~ k / sqrt(eps)
    k2 = k.copy()
    k2[0, 0, 0] = 1e-5 * unit(k[0, 0, 0])
    _, st = oracle_mod.gdn_fwd(q[:, :, :1], k2[:, :, :1], v[:, :, :1], a[:, :, :1], b[:, :, :1], None, eps=1e-6)
    kh = k2[0, 0, 0] / np.sqrt(1e-10 + 1e-6)
    np.testing.assert_allclose(st[0, 0], b[0, 0, 0] * np.outer(kh, v[0, 0, 0]), rtol=1e-12)


def test_empty_sequence_copies_state(oracle_mod):
    rng = np.random.default_rng(12)
    q, k, v, a, b, s = rand_case(rng, T=0, dk=4, dv=4)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    assert out.shape == (1, 1, 0, 4)
    np.testing.assert_array_equal(st, s)
    _, z = oracle_mod.gdn_fwd(q, k, v, a, b, None, eps=0.0)
    np.testing.assert_array_equal(z, np.zeros_like(s))


def test_nan_propagates(oracle_mod):
    rng = np.random.default_rng(13)
    q, k, v, a, b, s = rand_case(rng, T=5, dk=4, dv=4)
    v[0, 0, 2, 1] = np.nan
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s, eps=0.0)
    assert np.isnan(out[0, 0, 2, 1]) and np.isnan(st[0, 0, :, 1]).any()
    assert np.isfinite(out[0, 0, :2]).all()


# ------------------------------------------------------------ fused gates


def test_gate_maps_closed_forms(oracle_mod):
    """alpha = exp(-softplus(a)) is the logistic function of -a, beta = sigmoid(b):
    alpha(a) + beta(a) = 1 (exp(-log(1 + e^a)) = 1 / (1 + e^a)), sigmoid(0) = 1/2,
    and the tails: alpha -> 1 and beta -> e^b for b -> -inf, alpha -> e^-a for a -> +inf.
    A sign slip (softplus(-a), exp(+b)) or a dropped exp fails these."""
    x = np.array([-60.0, -30.0, -5.0, -1.0, -0.25, 0.0, 0.25, 1.0, 5.0, 30.0, 60.0])
    al, be = oracle_mod.gates(x, x)
    np.testing.assert_allclose(al + be, 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(al, 1.0 / (1.0 + np.exp(x)), rtol=1e-14, atol=0)
    assert be[x == 0.0][0] == 0.5 and al[x == 0.0][0] == 0.5
    np.testing.assert_allclose(be[:2], np.exp(x[:2]), rtol=1e-12)        # beta -> e^b
    np.testing.assert_allclose(al[-2:], np.exp(-x[-2:]), rtol=1e-12)     # alpha -> e^-a
    assert al[0] == 1.0 and be[-1] == 1.0
    # monotone: alpha decreasing, beta increasing
    assert np.all(np.diff(al) < 0) and np.all(np.diff(be) > 0)


def test_gate_logits_equal_gate_values(oracle_mod):
    """The recurrence from logits equals the recurrence from gate values formed
    by the logistic closed form alpha = 1 / (1 + e^a), beta = 1 / (1 + e^-b)."""
    rng = np.random.default_rng(41)
    q, k, v, _, _, s = rand_case(rng, B=2, H=2, T=40, dk=8, dv=7)
    za = rng.standard_normal(q.shape[:3]) * 2 - 1
    zb = rng.standard_normal(q.shape[:3])
    o1, s1 = oracle_mod.gdn_fwd(q, k, v, za, zb, s, gate_logits=True)
    o2, s2 = oracle_mod.gdn_fwd(q, k, v, 1.0 / (1.0 + np.exp(za)), 1.0 / (1.0 + np.exp(-zb)), s)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-12)


def test_output_gate_is_elementwise(oracle_mod):
    """g = 1 leaves the outputs unchanged, g = 0 zeroes them, and a general g
    scales each output element by itself; the state is not gated."""
    rng = np.random.default_rng(43)
    q, k, v, a, b, s = rand_case(rng, T=25, dk=6, dv=5)
    o0, s0 = oracle_mod.gdn_fwd(q, k, v, a, b, s)
    o1, s1 = oracle_mod.gdn_fwd(q, k, v, a, b, s, out_gate=np.ones_like(o0))
    oz, _ = oracle_mod.gdn_fwd(q, k, v, a, b, s, out_gate=np.zeros_like(o0))
    g = rng.uniform(0.0, 1.0, o0.shape)
    og, sg = oracle_mod.gdn_fwd(q, k, v, a, b, s, out_gate=g)
    assert np.array_equal(o1, o0) and np.array_equal(s1, s0)
    assert np.all(oz == 0.0)
    # element (t, j) of the gated output, written out from the definition
    for t in (0, 7, 24):
        for j in range(o0.shape[-1]):
            assert og[0, 0, t, j] == o0[0, 0, t, j] * g[0, 0, t, j]
    assert np.array_equal(sg, s0)


# ---- bidirectional scan (SANA-Streaming section 4.1: forward scan from the
# cache plus a backward scan within the chunk; section 2.3: both histories
# are combined for the output)

def _rev(x):
    return np.ascontiguousarray(np.asarray(x)[:, :, ::-1])


def test_bidir_time_reversal_symmetry(oracle_mod):
    """From a zero state the bidirectional output of the reversed sequence is
    the reversed output: the backward scan is the forward recurrence run over
    the tokens in reverse, each token with its own gates."""
    rng = np.random.default_rng(31)
    q, k, v, a, b, _ = rand_case(rng, B=2, H=2, T=23, dk=5, dv=4)
    out, _ = oracle_mod.gdn_bidir(q, k, v, a, b, None)
    out_r, _ = oracle_mod.gdn_bidir(_rev(q), _rev(k), _rev(v), _rev(a), _rev(b), None)
    np.testing.assert_allclose(_rev(out_r), out, rtol=1e-12, atol=1e-12)
    # and the two halves are not symmetric on their own
    fwd, _ = oracle_mod.gdn_fwd(q, k, v, a, b, None)
    assert np.abs(fwd - out).max() > 1e-3


def test_bidir_orthonormal_keys_both_sides(oracle_mod):
    """Orthonormal keys decouple the delta correction in both scans: with a
    zero state, o_t = sum_s w_ts beta_s (k_s . q_t) v_s with
    w_ts = prod_{r=s+1..t} alpha_r for s <= t (forward) plus
    prod_{r=t..s-1} alpha_r for s >= t (backward: moving from token s back to
    t applies the gates of tokens t .. s-1), so the diagonal counts twice."""
    rng = np.random.default_rng(32)
    T, dk, dv = 11, 16, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None] * rng.uniform(0.5, 2.0, size=(1, 1, T, 1))
    q = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    a = rng.uniform(0.3, 1.0, size=(1, 1, T))
    b = rng.uniform(0.0, 1.0, size=(1, 1, T))
    out, _ = oracle_mod.gdn_bidir(q, k, v, a, b, None, eps=0.0)
    al = a[0, 0]
    W = np.zeros((T, T))
    for t in range(T):
        for s in range(T):
            if s <= t:
                W[t, s] += np.prod(al[s + 1:t + 1])
            if s >= t:
                W[t, s] += np.prod(al[t:s])
    ref = (W * (unit(q[0, 0]) @ Qm[:T].T) * b[0, 0][None, :]) @ v[0, 0]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)


def test_bidir_small_beta_is_bidirectional_linear_attention(oracle_mod):
    """From a zero state and to first order in beta (any keys) the delta
    correction vanishes and the output is gated bidirectional linear
    attention with the weights of the orthonormal case (the error is second
    order in beta)."""
    rng = np.random.default_rng(33)
    T, dk, dv = 14, 6, 4
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    a = rng.uniform(0.4, 1.0, size=(1, 1, T))
    eps_b = 1e-4
    b = eps_b * rng.uniform(0.5, 1.0, size=(1, 1, T))
    out, _ = oracle_mod.gdn_bidir(q, k, v, a, b, None, eps=0.0)
    al = a[0, 0]
    W = np.zeros((T, T))
    for t in range(T):
        for s in range(T):
            if s <= t:
                W[t, s] += np.prod(al[s + 1:t + 1])
            if s >= t:
                W[t, s] += np.prod(al[t:s])
    qh, kh = unit(q[0, 0]), unit(k[0, 0])
    ref = (W * (qh @ kh.T) * b[0, 0][None, :]) @ v[0, 0]
    err = np.abs(out[0, 0] - ref).max()
    assert err < 10 * eps_b * np.abs(ref).max(), err
    assert np.abs(ref).max() > 0.5 * eps_b


def test_bidir_beta_zero_is_forward_decay(oracle_mod):
    """beta = 0: nothing is written, the backward scan (zero state) adds
    nothing and the output is the decayed incoming state read out."""
    rng = np.random.default_rng(34)
    q, k, v, a, _, s0 = rand_case(rng, T=9)
    z = np.zeros_like(a)
    out, st = oracle_mod.gdn_bidir(q, k, v, a, z, s0, eps=0.0)
    g = np.cumprod(a[0, 0])
    ref = g[:, None] * (unit(q[0, 0]) @ s0[0, 0])
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st[0, 0], g[-1] * s0[0, 0], rtol=1e-12, atol=1e-13)


# ---- softmax attention with a sink chunk and a recent window (SANA-Streaming
# section 2.1, "Softmax blocks for local window and sink refinement")

def _attn_case(rng, B=1, H=2, Nq=7, ns=5, nw=3, nc=6, d=8):
    r = lambda n: rng.standard_normal((B, H, n, d))
    return r(Nq), r(ns), r(ns), r(nw), r(nw), r(nc), r(nc)


def test_attn_zero_query_averages_values(oracle_mod):
    """q = 0 gives equal scores: every output row is the mean of all values."""
    rng = np.random.default_rng(41)
    q, ks, vs, kw, vw, kc, vc = _attn_case(rng)
    out = oracle_mod.attn_sink_window(np.zeros_like(q), ks, vs, kw, vw, kc, vc)
    mean = np.concatenate([vs, vw, vc], axis=2).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(out, np.broadcast_to(mean, out.shape), rtol=1e-13, atol=1e-13)


def test_attn_two_keys_closed_form(oracle_mod):
    """Two keys: the weight of the first is the logistic function of the
    scaled score difference."""
    rng = np.random.default_rng(42)
    d = 4
    q = rng.standard_normal((1, 1, 3, d))
    k1, k2 = rng.standard_normal((1, 1, 1, d)), rng.standard_normal((1, 1, 1, d))
    v1, v2 = rng.standard_normal((1, 1, 1, d)), rng.standard_normal((1, 1, 1, d))
    e = np.zeros((1, 1, 0, d))
    out = oracle_mod.attn_sink_window(q, k1, v1, e, e, k2, v2, scale=0.7)
    w = 1.0 / (1.0 + np.exp(-0.7 * (q[0, 0] @ (k1 - k2)[0, 0, 0])))
    ref = w[:, None] * v1[0, 0, 0] + (1 - w)[:, None] * v2[0, 0, 0]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_attn_split_by_log_sum_exp(oracle_mod):
    """Attention over [A; B] equals the attentions over A and over B mixed by
    their softmax masses, exp(lse_A) : exp(lse_B) (the identity that lets a
    kernel walk the context in tiles)."""
    rng = np.random.default_rng(43)
    q, ks, vs, kw, vw, kc, vc = _attn_case(rng, d=6)
    e = np.zeros_like(kw[:, :, :0])
    s = 1.0 / np.sqrt(6)
    full = oracle_mod.attn_sink_window(q, ks, vs, kw, vw, kc, vc)
    oa = oracle_mod.attn_sink_window(q, ks, vs, e, e, e, e)
    ob = oracle_mod.attn_sink_window(q, e, e, kw, vw, kc, vc)
    la = np.log(np.exp(s * q @ np.swapaxes(ks, 2, 3)).sum(-1, keepdims=True))
    kb = np.concatenate([kw, kc], axis=2)
    lb = np.log(np.exp(s * q @ np.swapaxes(kb, 2, 3)).sum(-1, keepdims=True))
    wa = 1.0 / (1.0 + np.exp(lb - la))
    np.testing.assert_allclose(full, wa * oa + (1 - wa) * ob, rtol=1e-12, atol=1e-13)


def test_attn_key_permutation_and_segment_placement(oracle_mod):
    """The output does not depend on the order of the (key, value) pairs nor
    on which of the three segments holds them."""
    rng = np.random.default_rng(44)
    q, ks, vs, kw, vw, kc, vc = _attn_case(rng)
    out = oracle_mod.attn_sink_window(q, ks, vs, kw, vw, kc, vc)
    K = np.concatenate([ks, kw, kc], axis=2)
    V = np.concatenate([vs, vw, vc], axis=2)
    perm = rng.permutation(K.shape[2])
    e = K[:, :, :0]
    out2 = oracle_mod.attn_sink_window(q, e, e, K[:, :, perm[:4]], V[:, :, perm[:4]],
                                       K[:, :, perm[4:]], V[:, :, perm[4:]])
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)


def test_attn_matches_library_attention(oracle_mod):
    """Against torch's scaled_dot_product_attention on the CPU in fp64 (an
    independent implementation), with large scores to exercise the max shift."""
    import torch
    rng = np.random.default_rng(45)
    q, ks, vs, kw, vw, kc, vc = _attn_case(rng, B=2, H=3, Nq=9, ns=4, nw=5, nc=9, d=16)
    q = q * 4.0
    out = oracle_mod.attn_sink_window(q, ks, vs, kw, vw, kc, vc)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    K = torch.cat([t(ks), t(kw), t(kc)], dim=2)
    V = torch.cat([t(vs), t(vw), t(vc)], dim=2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), K, V).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


# ---- frame-wise GDN with a normalised readout (SANA-Streaming section 2.1,
# "Frame-wise Gated DeltaNet": one state update per frame rather than per
# token; section 2.3: frame summaries, a scan over frames, the frame's queries
# read against its state; appendix G.3-G.5): the frame's mean of the delta
# rule's writes and erasures, one decay per frame, a denominator state driven
# by a value of constant 1, output = numerator / denominator, then the gate

def _frame_case(rng, B=1, H=2, F=3, N=5, dk=6, dv=4, state=True):
    T = F * N
    q = np.abs(rng.standard_normal((B, H, T, dk)))     # non-negative features
    k = np.abs(rng.standard_normal((B, H, T, dk)))
    v = rng.standard_normal((B, H, T, dv))
    a = np.exp(-np.log1p(np.exp(rng.standard_normal((B, H, F)))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    s = rng.standard_normal((B, H, dk, dv)) * 0.3 if state else None
    z = np.abs(rng.standard_normal((B, H, dk))) * 0.5 + 0.2 if state else None
    return q, k, v, a, b, s, z


def test_framewise_one_token_frames_are_the_tokenwise_rule(oracle_mod):
    """N = 1: every frame is one token, and the frame-wise update is the
    token-wise gated delta rule of the C oracle (an independent token loop):
    numerator = its scan over v, denominator = its scan over a value column of
    ones from z_in, out = numerator / denominator * gate."""
    rng = np.random.default_rng(51)
    q, k, v, a, b, s, z = _frame_case(rng, F=7, N=1)
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal(v.shape)))
    out, s_out, z_out = oracle_mod.gdn_framewise(q, k, v, a, b, 1, s, z, out_gate=g)
    num, s_ref = oracle_mod.gdn_fwd(q, k, v, a, b, s)
    den, z_ref = oracle_mod.gdn_fwd(q, k, np.ones(v.shape[:-1] + (1,)), a, b, z[..., None])
    np.testing.assert_allclose(out, num / den * g, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s_out, s_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z_out, z_ref[..., 0], rtol=1e-12, atol=1e-13)


def test_framewise_orthonormal_frame_keys_equal_sequential_writes(oracle_mod):
    """Keys orthonormal within each frame: the frame's token writes commute
    and do not interfere, so one frame update with beta equals the token-wise
    scan (C oracle) over the frame's tokens with beta / N and the frame decay
    on its first token.  The states agree at every frame end, and so does the
    output of each frame's last token, which reads the state after the whole
    frame in both."""
    rng = np.random.default_rng(57)
    F, N, dk, dv = 4, 5, 8, 3
    k = np.empty((1, 2, F * N, dk))
    for h in range(2):
        for f in range(F):
            Qo, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
            k[0, h, f * N:(f + 1) * N] = Qo[:N]
    q = np.abs(rng.standard_normal((1, 2, F * N, dk)))
    v = rng.standard_normal((1, 2, F * N, dv))
    a = rng.uniform(0.3, 1.0, (1, 2, F))
    b = rng.uniform(0.0, 1.0, (1, 2, F * N))
    s = rng.standard_normal((1, 2, dk, dv)) * 0.4
    z = np.abs(rng.standard_normal((1, 2, dk))) + 0.3
    out, s_out, z_out = oracle_mod.gdn_framewise(q, k, v, a, b, N, s, z)
    a_tok = np.ones(b.shape)
    a_tok[:, :, ::N] = a
    num, s_ref = oracle_mod.gdn_fwd(q, k, v, a_tok, b / N, s)
    den, z_ref = oracle_mod.gdn_fwd(q, k, np.ones(v.shape[:-1] + (1,)), a_tok, b / N, z[..., None])
    last = np.arange(N - 1, F * N, N)
    np.testing.assert_allclose(out[:, :, last], (num / den)[:, :, last], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s_out, s_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z_out, z_ref[..., 0], rtol=1e-12, atol=1e-13)


def test_framewise_is_one_gradient_step_on_the_frame_loss(oracle_mod):
    """The reading as its definition: S_f is one gradient step, of unit size,
    on L(S) = (1/N) sum_n beta_n ||S k_n - v_n||^2 / 2 taken from the decayed
    state alpha_f S_{f-1}; the gradient comes from torch autograd in fp64, an
    independent route to the same update (likewise z with values 1)."""
    import torch
    rng = np.random.default_rng(58)
    q, k, v, a, b, s, z = _frame_case(rng, B=1, H=1, F=3, N=6, dk=5, dv=3)
    N, F = 6, 3
    kh = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)      # the oracle's eps (pinned above)
    S = torch.tensor(s[0, 0].T.copy(), dtype=torch.float64)       # S = M^T  [dv][dk]
    Z = torch.tensor(z[0, 0].copy(), dtype=torch.float64)          # [dk]
    for f in range(F):
        K = torch.tensor(kh[0, 0, f * N:(f + 1) * N])
        V = torch.tensor(v[0, 0, f * N:(f + 1) * N])
        be = torch.tensor(b[0, 0, f * N:(f + 1) * N])
        S0 = (a[0, 0, f] * S).clone().requires_grad_(True)
        loss = 0.5 * (be[:, None] * (K @ S0.T - V) ** 2).sum() / N
        loss.backward()
        S = (S0 - S0.grad).detach()
        Z0 = (a[0, 0, f] * Z).clone().requires_grad_(True)
        lz = 0.5 * (be * (K @ Z0 - 1.0) ** 2).sum() / N
        lz.backward()
        Z = (Z0 - Z0.grad).detach()
    _, s_out, z_out = oracle_mod.gdn_framewise(q, k, v, a, b, N, s, z)
    np.testing.assert_allclose(s_out[0, 0], S.numpy().T, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z_out[0, 0], Z.numpy(), rtol=1e-12, atol=1e-13)


def test_framewise_beta_zero_readout_is_decay_free(oracle_mod):
    """beta = 0: nothing is written, both states only decay by the product of
    the frames' alphas, and the decay cancels in the ratio: every output is
    (M_in^T q^) / (z_in . q^)."""
    rng = np.random.default_rng(52)
    q, k, v, a, b, s, z = _frame_case(rng)
    out, s_out, z_out = oracle_mod.gdn_framewise(q, k, v, a, np.zeros_like(b), q.shape[2] // a.shape[-1], s, z)
    qh = unit(q)
    ref = np.einsum("bhij,bhti->bhtj", s, qh) / np.einsum("bhi,bhti->bht", z, qh)[..., None]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    pa = a.prod(axis=-1)
    np.testing.assert_allclose(s_out, pa[..., None, None] * s, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(z_out, pa[..., None] * z, rtol=1e-13, atol=1e-15)


def test_framewise_token_order_inside_a_frame_does_not_matter(oracle_mod):
    """A frame is updated at once: permuting the tokens inside each frame
    permutes their outputs the same way and leaves both states unchanged
    (the token-sequential reading fails this)."""
    rng = np.random.default_rng(59)
    q, k, v, a, b, s, z = _frame_case(rng, F=3, N=6)
    N, F = 6, 3
    perm = np.concatenate([f * N + rng.permutation(N) for f in range(F)])
    o1, s1, z1 = oracle_mod.gdn_framewise(q, k, v, a, b, N, s, z)
    o2, s2, z2 = oracle_mod.gdn_framewise(q[:, :, perm], k[:, :, perm], v[:, :, perm], a, b[:, :, perm],
                                          N, s, z)
    np.testing.assert_allclose(o2, o1[:, :, perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z2, z1, rtol=1e-12, atol=1e-13)


def test_framewise_repeated_token_equals_one_token(oracle_mod):
    """A frame of N copies of one token (same k, v, beta) has the mean of N
    equal terms: it equals a one-token frame of that token."""
    rng = np.random.default_rng(60)
    q1, k1, v1, a, b1, s, z = _frame_case(rng, F=3, N=1)
    N = 4
    rep = lambda x: np.repeat(x, N, axis=2)
    qN = np.abs(rng.standard_normal(rep(q1).shape))
    o1, s1, z1 = oracle_mod.gdn_framewise(q1, k1, v1, a, b1, 1, s, z)
    oN, sN, zN = oracle_mod.gdn_framewise(qN, rep(k1), rep(v1), a, rep(b1), N, s, z)
    np.testing.assert_allclose(sN, s1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(zN, z1, rtol=1e-12, atol=1e-13)
    qh = unit(qN)
    ref = np.einsum("bhfij,bhfni->bhfnj", np.stack([oracle_mod.gdn_framewise(
        q1[:, :, :f + 1], k1[:, :, :f + 1], v1[:, :, :f + 1], a[:, :, :f + 1], b1[:, :, :f + 1], 1, s, z)[1]
        for f in range(3)], axis=2), qh.reshape(1, 2, 3, N, -1))
    den = np.einsum("bhfi,bhfni->bhfn", np.stack([oracle_mod.gdn_framewise(
        q1[:, :, :f + 1], k1[:, :, :f + 1], v1[:, :, :f + 1], a[:, :, :f + 1], b1[:, :, :f + 1], 1, s, z)[2]
        for f in range(3)], axis=2), qh.reshape(1, 2, 3, N, -1))
    np.testing.assert_allclose(oN, (ref / den[..., None]).reshape(oN.shape), rtol=1e-11, atol=1e-12)


def test_framewise_contraction_bound(oracle_mod):
    """beta in [0, 1] and unit keys: I - G_f has eigenvalues in [0, 1], so
    ||M_f||_2 <= alpha_f ||M_{f-1}||_2 + max_n ||v_n|| for frames of 880
    tokens (a frame-sized write would blow up with the plain sum)."""
    rng = np.random.default_rng(61)
    q, k, v, a, b, s, z = _frame_case(rng, B=1, H=1, F=1, N=880, dk=16, dv=8)
    norm2 = lambda m: np.linalg.norm(m, 2)
    M = s[0, 0]
    for f in range(5):
        qf, kf, vf = (rng.standard_normal(x.shape) for x in (q, k, v))
        bf = rng.uniform(0, 1, b.shape)
        _, s_out, _ = oracle_mod.gdn_framewise(np.abs(qf), kf, vf, a, bf, 880, M[None, None], z)
        bound = a[0, 0, 0] * norm2(M) + np.linalg.norm(vf[0, 0], axis=-1).max()
        assert norm2(s_out[0, 0]) <= bound * (1 + 1e-12)
        M = s_out[0, 0]


def test_framewise_constant_values_read_back(oracle_mod):
    """From zero states, a value that is the same vector c at every token
    drives every numerator column as c_j times the denominator: out = c."""
    rng = np.random.default_rng(53)
    q, k, v, a, b, _, _ = _frame_case(rng, state=False)
    c = rng.standard_normal(v.shape[-1])
    out, _, _ = oracle_mod.gdn_framewise(q, k, np.broadcast_to(c, v.shape), a, b, q.shape[2] // a.shape[-1])
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=1e-11, atol=1e-12)


def test_framewise_shift_equivariance(oracle_mod):
    """Adding c to every value, and z_in c^T to the numerator state, adds c to
    every output (the normalised readout is an affine average of values)."""
    rng = np.random.default_rng(54)
    q, k, v, a, b, s, z = _frame_case(rng)
    N = q.shape[2] // a.shape[-1]
    c = rng.standard_normal(v.shape[-1])
    o1, s1, z1 = oracle_mod.gdn_framewise(q, k, v, a, b, N, s, z)
    o2, s2, z2 = oracle_mod.gdn_framewise(q, k, v + c, a, b, N, s + z[..., None] * c, z)
    np.testing.assert_allclose(o2, o1 + c, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s2, s1 + z1[..., None] * c, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(z2, z1, rtol=0, atol=0)


def test_framewise_split_across_calls(oracle_mod):
    """Frames F1 then F - F1 in two calls with both states carried equal one
    call over all F frames."""
    rng = np.random.default_rng(56)
    q, k, v, a, b, s, z = _frame_case(rng, F=4, N=3)
    N, F1 = 3, 1
    cut = F1 * N
    o, s_out, z_out = oracle_mod.gdn_framewise(q, k, v, a, b, N, s, z)
    o1, s1, z1 = oracle_mod.gdn_framewise(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], a[:, :, :F1],
                                          b[:, :, :cut], N, s, z)
    o2, s2, z2 = oracle_mod.gdn_framewise(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], a[:, :, F1:],
                                          b[:, :, cut:], N, s1, z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, s_out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(z2, z_out, rtol=1e-13, atol=1e-14)


def test_attn_score_shift_invariance_and_value_shift(oracle_mod):
    """Adding the same vector u to every key moves all scores of a query by
    scale * (q . u), which the softmax ignores; adding c to every value adds
    c to every output (the weights sum to one)."""
    rng = np.random.default_rng(46)
    q, ks, vs, kw, vw, kc, vc = _attn_case(rng, d=8)
    out = oracle_mod.attn_sink_window(q, ks, vs, kw, vw, kc, vc)
    u = 3.0 * rng.standard_normal(8)
    out_k = oracle_mod.attn_sink_window(q, ks + u, vs, kw + u, vw, kc + u, vc)
    np.testing.assert_allclose(out_k, out, rtol=1e-11, atol=1e-12)
    c = rng.standard_normal(8)
    out_v = oracle_mod.attn_sink_window(q, ks, vs + c, kw, vw + c, kc, vc + c)
    np.testing.assert_allclose(out_v, out + c, rtol=1e-11, atol=1e-12)
