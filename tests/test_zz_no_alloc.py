"""gdn_fwd_step_noalloc (scratch in the library's static device array) against
gdn_fwd_step (scratch from a workspace the caller allocates): the same
kernels on the same launch plan, so the outputs and states must be equal bit
for bit, on two calls in a row, the second with a smaller input (the array
keeps the first call's contents), and both meet the oracle's bar.  Also: a
shape whose plan needs more scratch than the array holds is refused before
any launch."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call, to_numpy64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,first,second", [
    ("rollout_h16_d128", dict(H=16, T=2640), dict(H=5, T=700)),       # segmented plan, then a smaller one
    ("stream_chunk_h16_d64", dict(H=16, T=2640), dict(H=3, T=333)),
    # 48 heads of one frame: two segments, the largest scratch of the workloads
    ("frame_step_b2_h24_d128", dict(B=2, H=24, T=880), dict(B=1, H=20, T=640)),
])
def test_noalloc_equals_step_on_two_calls(gdn_lib, oracle_mod, wl_name, first, second):
    wl = WORKLOADS[wl_name]
    for i, shape in enumerate((first, second)):
        announce(f"noalloc {wl_name} call {i} {shape}")
        d = make_call(wl, i, **shape)
        g = to_dev(d)
        args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
        o_ref, s_ref = gdn_lib.fwd_step(*args)
        o_na, s_na = gdn_lib.fwd_step_noalloc(*args)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref), "outputs differ from gdn_fwd_step"
        assert torch.equal(s_na, s_ref), "states differ from gdn_fwd_step"
        ro, rs = oracle_mod.gdn_fwd(*(to_numpy64(d[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                    None if d["state_in"] is None else to_numpy64(d["state_in"]))
        assert_close(o_na.to("cpu", torch.float64).numpy(), ro, False, "noalloc out")
        assert_close(s_na.to("cpu", torch.float64).numpy(), rs, False, "noalloc state")


def test_noalloc_refuses_shapes_beyond_its_scratch(gdn_lib):
    lib = gdn_lib.load()
    cap = 64 << 20
    # find a few-head shape whose segmented plan needs more than the array
    B, H, T, dk, dv = 1, 64, 8192, 128, 128
    need = gdn_lib.workspace_bytes(B, H, T, dk, dv, 0)
    if need <= cap:
        pytest.skip(f"plan of the probe shape needs only {need} bytes")
    announce(f"noalloc refusal need={need}")
    q = torch.zeros(B, H, T, dk, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(B, H, T, dv, dtype=torch.bfloat16, device="cuda")
    a = torch.ones(B, H, T, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn_lib.GdnError, match="scratch"):
        gdn_lib.fwd_step_noalloc(q, q, v, a, a)
