"""GPU parity under rescaling of v and the state.

The gated delta rule is linear in (v, S): scaling v and the incoming state by
the same factor scales every output and the outgoing state by that factor,
and the fp64 oracle is exactly homogeneous.  Powers of two keep the scaled
bf16 v and fp32 state exact, so the HIP path must meet the same bar at every
scale: rel-L2 2e-3, and max-abs 2e-2 times the scale.  Each kernel family that
serves bf16 inputs is covered: the segmented walk with its correction pass
(16 heads, 42 chunks), the unsegmented walk (48 heads), the single-pass
kernel of 128-token chunks, and the walker of d_k = 32 heads.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_BF16, announce, errors, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call, to_numpy64

pytestmark = pytest.mark.gpu

SCALES = [2.0 ** -16, 2.0 ** -8, 2.0 ** 8, 2.0 ** 12]

# (label, workload, overrides of make_call, api, chunk); "walker32" runs the
# walker of d_k = 32 heads (gdn_fwd.hip: a summary pass and a main pass)
PATHS = [
    ("segmented", "stream_chunk_h16_d64", {}, "step", None),
    ("unsegmented", "frame_step_b2_h24_d128", {}, "step", None),
    ("chunk128", "stream_chunk_h16_d64", {"H": 4}, "chunked", 128),
    ("walker32", "stream_chunk_h16_d64", {"H": 4, "dk": 32}, "chunked", 64),
]


def _scaled(d, s):
    out = dict(d)
    out["v"] = (d["v"].to(torch.float32) * s).to(d["v"].dtype)
    assert torch.equal(out["v"].to(torch.float32), d["v"].to(torch.float32) * s)
    if d["state_in"] is not None:
        out["state_in"] = d["state_in"] * s
    return out


def _bar(got, ref, s, what):
    maxabs, rel = errors(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert rel <= TOL_BF16["rel"], f"{what}: rel-L2 {rel:.3e}"
    assert maxabs <= TOL_BF16["maxabs"] * s, f"{what}: max-abs {maxabs:.3e} > {TOL_BF16['maxabs'] * s:.3e}"
    return maxabs, rel


@pytest.mark.parametrize("scale", SCALES, ids=["2^-16", "2^-8", "2^8", "2^12"])
@pytest.mark.parametrize("label,wname,over,api,chunk", PATHS, ids=[p[0] for p in PATHS])
def test_homogeneous_in_v_and_state(gdn_lib, oracle_mod, label, wname, over, api, chunk, scale):
    wl = WORKLOADS[wname]
    over = dict(over)
    if "dk" in over:
        wl = wl.replace(dk=over.pop("dk"))
    d = make_call(wl, 0, **over)
    if d["state_in"] is None:
        d["state_in"] = torch.randn(d["v"].shape[0], d["v"].shape[1], wl.dk, wl.dv,
                                    generator=torch.Generator().manual_seed(7)) * 0.02
    ds = _scaled(d, scale)
    announce(f"scale {label} {wname} {over} api={api} chunk={chunk} scale={scale}")
    g = to_dev(ds)
    if api == "step":
        o, s_out = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
    else:
        o, s_out = gdn_lib.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], chunk)
    torch.cuda.synchronize()
    o = o.to("cpu", torch.float64).numpy()
    s_out = s_out.to("cpu", torch.float64).numpy()
    ref_o, ref_s = oracle_mod.gdn_fwd(*(to_numpy64(ds[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                      to_numpy64(ds["state_in"]))
    r1 = _bar(o, ref_o, scale, f"{label} x{scale} out")
    r2 = _bar(s_out, ref_s, scale, f"{label} x{scale} state")
    print(f"   out maxabs/scale {r1[0] / scale:.2e} rel {r1[1]:.2e} | state maxabs/scale "
          f"{r2[0] / scale:.2e} rel {r2[1]:.2e}", flush=True)
