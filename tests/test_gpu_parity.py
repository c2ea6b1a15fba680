"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, for the five workloads (reduced sizes
that span several tiles and a ragged tail, and full sizes on every head),
the chunk sizes 32/64/128, and the edge cases of the method."""
import numpy as np
import pytest
import torch

from gpu_helpers import (announce, assert_close, gpu_rollout, oracle_rollout, select_heads,
                         to_dev)
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call

pytestmark = pytest.mark.gpu


def _check_rollout(gdn, oracle, wl, calls, *, B=None, H=None, T=None, chunk=None, api="chunked",
                   heads=None, out_dtype=torch.float32, what=""):
    announce(f"{what} {wl.name} calls={calls} B={B or wl.B} H={H or wl.H} T={T or wl.T} "
             f"chunk={chunk or wl.chunk} api={api} heads={heads}")
    g_outs, g_state, ins = gpu_rollout(gdn, wl, calls, B=B, H=H, T=T, chunk=chunk, api=api,
                                       out_dtype=out_dtype)
    o_outs, o_state = oracle_rollout(oracle, ins, heads)
    if heads is not None:
        g_outs = [select_heads(o, heads) for o in g_outs]
        g_state = select_heads(g_state, heads)
    f32 = wl.dtype == "f32"
    r1 = assert_close(np.concatenate(g_outs, 2), np.concatenate(o_outs, 2), f32, what + " out")
    r2 = assert_close(g_state, o_state, f32, what + " state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state maxabs {r2[0]:.2e} rel {r2[1]:.2e}",
          flush=True)
    return g_outs, g_state


# ------------------------------------------------------------ the workloads


@pytest.mark.parametrize("chunk", [32, 64])
def test_tiny_fp32(gdn_lib, oracle_mod, chunk):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["tiny_f32"], 1, chunk=chunk, what="tiny")


@pytest.mark.parametrize("api", ["chunked", "step"])
def test_stream_chunk_full(gdn_lib, oracle_mod, api):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["stream_chunk_h16_d64"], 1, api=api,
                   what="stream")


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_stream_chunk_sizes(gdn_lib, oracle_mod, chunk):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["stream_chunk_h16_d64"], 1, H=4, chunk=chunk,
                   what="stream-chunk")


def test_rollout_reduced(gdn_lib, oracle_mod):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["rollout_h16_d128"], 3, H=3, api="step",
                   what="rollout-reduced")


def test_rollout_full_all_heads(gdn_lib, oracle_mod):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["rollout_h16_d128"], 20, api="step",
                   what="rollout-full")


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_prefill_reduced(gdn_lib, oracle_mod, chunk):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["prefill_b4_h32_d128"], 1, B=2, H=2, T=1000,
                   chunk=chunk, what="prefill-reduced")


def test_prefill_full_all_heads(gdn_lib, oracle_mod):
    wl = WORKLOADS["prefill_b4_h32_d128"]
    ins = [make_call(wl, 0)]
    announce("prefill-full oracle, all 128 heads")
    o_outs, o_state = oracle_rollout(oracle_mod, ins)
    for chunk in (32, 64, 128):
        announce(f"prefill-full chunk={chunk}")
        g_outs, g_state, _ = gpu_rollout(gdn_lib, wl, 1, chunk=chunk, inputs=ins)
        r1 = assert_close(g_outs[0], o_outs[0], False, f"prefill C={chunk} out")
        r2 = assert_close(g_state, o_state, False, f"prefill C={chunk} state")
        print(f"   C={chunk} out {r1} state {r2}", flush=True)
        del g_outs, g_state


def test_frame_step_reduced(gdn_lib, oracle_mod):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["frame_step_b2_h24_d128"], 8, B=1, H=3,
                   api="step", what="frame-reduced")


def test_frame_step_full_all_heads(gdn_lib, oracle_mod):
    _check_rollout(gdn_lib, oracle_mod, WORKLOADS["frame_step_b2_h24_d128"], 200, api="step",
                   what="frame-full")


# ------------------------------------------------------------- edge cases

EDGE = WORKLOADS["stream_chunk_h16_d64"]


@pytest.mark.parametrize("T", [1, 15, 63, 64, 65, 129])
def test_ragged_lengths(gdn_lib, oracle_mod, T):
    _check_rollout(gdn_lib, oracle_mod, EDGE, 1, H=2, T=T, what=f"T={T}")


def test_empty_sequence_copies_state(gdn_lib):
    d = to_dev(make_call(EDGE, 0, H=2, T=4))
    s_in = d["state_in"]
    e = lambda t: t[:, :, :0].contiguous()
    announce("T=0")
    out, s = gdn_lib.fwd_chunked(e(d["q"]), e(d["k"]), e(d["v"]), e(d["alpha"]), e(d["beta"]), s_in, 64)
    torch.cuda.synchronize()
    assert out.shape[2] == 0
    assert torch.equal(s, s_in)
    _, z = gdn_lib.fwd_chunked(e(d["q"]), e(d["k"]), e(d["v"]), e(d["alpha"]), e(d["beta"]), None, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0


@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 128), (128, 32), (128, 64), (32, 32)])
def test_head_shapes(gdn_lib, oracle_mod, dk, dv):
    wl = EDGE.replace(dk=dk, dv=dv)
    _check_rollout(gdn_lib, oracle_mod, wl, 1, H=3, T=300, what=f"dk={dk} dv={dv}")


def _custom(gdn, oracle, d, what, chunk=64, f32=False):
    announce(what)
    g = to_dev(d)
    o, s = gdn.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], chunk)
    torch.cuda.synchronize()
    ro, rs = oracle_rollout(oracle, [d])
    assert_close(o.double().cpu().numpy(), ro[0], f32, what + " out")
    assert_close(s.double().cpu().numpy(), rs, f32, what + " state")


def test_beta_zero_and_alpha_one(gdn_lib, oracle_mod):
    d = make_call(EDGE, 0, H=2, T=200)
    d["beta"] = torch.zeros_like(d["beta"])
    _custom(gdn_lib, oracle_mod, d, "beta=0")
    d = make_call(EDGE, 0, H=2, T=200)
    d["alpha"] = torch.ones_like(d["alpha"])
    _custom(gdn_lib, oracle_mod, d, "alpha=1")


def test_collinear_keys_full_write(gdn_lib, oracle_mod):
    """Identical keys with alpha = beta = 1: the worst-conditioned triangular solve."""
    d = make_call(EDGE, 0, H=2, T=200)
    d["k"] = d["k"][:, :, :1].expand_as(d["k"]).contiguous()
    d["alpha"] = torch.ones_like(d["alpha"])
    d["beta"] = torch.ones_like(d["beta"])
    _custom(gdn_lib, oracle_mod, d, "collinear")


def test_strong_decay(gdn_lib, oracle_mod):
    """alpha ~ 2^-10: cumulative log-decay far below fp32 exp range inside a chunk."""
    d = make_call(EDGE, 0, H=2, T=300)
    d["alpha"] = torch.full_like(d["alpha"], 2.0 ** -10)
    _custom(gdn_lib, oracle_mod, d, "strong-decay", chunk=128)


def test_correlated_keys(gdn_lib, oracle_mod):
    """Keys close to a shared direction (normalise(base + 0.1 noise)), as
    spatially correlated video tokens would be."""
    d = make_call(WORKLOADS["rollout_h16_d128"], 0, H=2, T=500)
    kf = d["k"].float()
    base = kf[:, :, :1]
    kk = base + 0.1 * torch.randn(kf.shape, generator=torch.Generator().manual_seed(5))
    d["k"] = (kk / kk.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    _custom(gdn_lib, oracle_mod, d, "correlated")


def test_bf16_output(gdn_lib, oracle_mod):
    _check_rollout(gdn_lib, oracle_mod, EDGE, 1, H=4, out_dtype=torch.bfloat16, what="bf16-out")


def test_zero_state_pointer_equals_zeros(gdn_lib):
    d = to_dev(make_call(WORKLOADS["rollout_h16_d128"], 0, H=2, T=300))
    announce("null-state")
    o1, s1 = gdn_lib.fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, 64)
    z = torch.zeros(1, 2, 128, 128, device="cuda")
    o2, s2 = gdn_lib.fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], z, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_in_place_state_and_determinism(gdn_lib):
    d = to_dev(make_call(EDGE, 0, H=3, T=700))
    announce("in-place")
    o1, s1 = gdn_lib.fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state_in"], 64)
    o2, s2 = gdn_lib.fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state_in"], 64)
    st = d["state_in"].clone()
    o3, s3 = gdn_lib.fwd_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "run-to-run results differ"
    assert torch.equal(st, s1) and torch.equal(o3, o1)


def test_split_invariance(gdn_lib, oracle_mod):
    """One call over T tokens vs two calls with the state carried."""
    d = make_call(EDGE, 0, H=2, T=1000)
    g = to_dev(d)
    announce("split")
    o, s = gdn_lib.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], 64)
    cut = 437
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, s1 = gdn_lib.fwd_chunked(*(part(g[n], 0, cut) for n in ("q", "k", "v", "alpha", "beta")),
                                 g["state_in"], 64)
    o2, s2 = gdn_lib.fwd_chunked(*(part(g[n], cut, 1000) for n in ("q", "k", "v", "alpha", "beta")),
                                 s1, 64)
    torch.cuda.synchronize()
    ro, rs = oracle_rollout(oracle_mod, [d])
    assert_close(torch.cat([o1, o2], 2).double().cpu().numpy(), ro[0], False, "split out")
    assert_close(s2.double().cpu().numpy(), rs, False, "split state")
    assert_close(o.double().cpu().numpy(), ro[0], False, "whole out")


def test_nan_stays_in_its_head(gdn_lib):
    d = to_dev(make_call(EDGE, 0, H=3, T=200))
    d["v"][0, 1, 50, 3] = float("nan")
    announce("nan")
    o, s = gdn_lib.fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state_in"], 64)
    torch.cuda.synchronize()
    assert torch.isfinite(o[0, 0]).all() and torch.isfinite(o[0, 2]).all()
    assert torch.isnan(o[0, 1]).any()


@pytest.mark.parametrize("name", ["stream_chunk_h16_d64", "rollout_h16_d128"])
def test_unsplit_walk_without_workspace(gdn_lib, oracle_mod, name):
    """Without a workspace every sequence is walked unsplit; both launch plans
    must match the oracle (and each other to rounding)."""
    wl = WORKLOADS[name]
    d = make_call(wl, 0, H=4)
    g = to_dev(d)
    announce(f"no-workspace {name}")
    o1, s1 = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"],
                              workspace=False)
    o2, s2 = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
    torch.cuda.synchronize()
    ro, rs = oracle_rollout(oracle_mod, [d])
    for o, s, what in ((o1, s1, "unsplit"), (o2, s2, "segmented")):
        assert_close(o.double().cpu().numpy(), ro[0], False, what + " out")
        assert_close(s.double().cpu().numpy(), rs, False, what + " state")


@pytest.mark.parametrize("dk,chunk", [(64, 64), (128, 64), (128, 32)])
def test_fp32_inputs_head_sizes(gdn_lib, oracle_mod, dk, chunk):
    """fp32 inputs beyond the tiny workload (dk = 128 runs the single-pass kernel)."""
    wl = WORKLOADS["tiny_f32"].replace(dk=dk, dv=dk)
    _check_rollout(gdn_lib, oracle_mod, wl, 1, H=2, T=300, chunk=chunk, what=f"f32 dk={dk}")


def test_resume_from_a_host_copy_of_the_state_is_bitwise(gdn_lib):
    # 20 carried calls straight, against the same calls with the state copied
    # to host memory after call 10 and loaded back into a fresh device buffer:
    # outputs and final state identical bit for bit
    wl = WORKLOADS["rollout_h16_d128"]
    announce("resume from host copy, rollout H=4, 20 calls")
    ins = [to_dev(make_call(wl, c, H=4)) for c in range(20)]
    outs_a, state = [], None
    for c, g in enumerate(ins):
        o, state = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state)
        outs_a.append(o)
    torch.cuda.synchronize()
    outs_b, state_b = [], None
    for c, g in enumerate(ins):
        o, state_b = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state_b)
        outs_b.append(o)
        if c == 9:
            torch.cuda.synchronize()
            host = state_b.to("cpu")
            del state_b
            state_b = host.to("cuda").contiguous()
    torch.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        assert torch.equal(a, b)
    assert torch.equal(state, state_b)
