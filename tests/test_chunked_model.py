"""The chunk-level (UT / WY) algebra evaluated by the GPU kernels, restated in
numpy fp64 (tests/chunked_model.py), must equal the token-by-token oracle to
fp64 rounding for every chunk length and ragged tail: this pins the
derivation itself, independently of any kernel."""
import numpy as np
import pytest

from chunked_model import chunked_fwd
from test_oracle_pins import rand_case


@pytest.mark.parametrize("C", [16, 32, 64, 128])
@pytest.mark.parametrize("T", [1, 15, 64, 100, 257])
def test_chunked_equals_oracle(oracle_mod, C, T):
    rng = np.random.default_rng(100 + C + T)
    q, k, v, a, b, s = rand_case(rng, B=1, H=2, T=T, dk=16, dv=8)
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s)
    oc, sc = chunked_fwd(q, k, v, a, b, s, C)
    np.testing.assert_allclose(oc, out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sc, st, rtol=1e-11, atol=1e-12)


def test_chunked_strong_decay_no_overflow(oracle_mod):
    """alpha ~ 1e-3 makes the cumulative log-decay reach -900 within a chunk;
    only non-positive exponents may be formed."""
    rng = np.random.default_rng(7)
    q, k, v, a, b, s = rand_case(rng, T=200, dk=8, dv=8)
    a[:] = 1e-3
    a[0, 0, 50:60] = 1.0
    out, st = oracle_mod.gdn_fwd(q, k, v, a, b, s)
    with np.errstate(over="raise", invalid="raise"):
        oc, sc = chunked_fwd(q, k, v, a, b, s, 128)
    np.testing.assert_allclose(oc, out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sc, st, rtol=1e-11, atol=1e-12)
