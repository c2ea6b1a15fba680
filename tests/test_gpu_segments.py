"""GPU parity of the segmented plan's edges, on every head, against the fp64
oracle: plain calls whose segment 0 walks from the incoming state and writes
its outputs itself, the correction pass that starts from segment 1 and splits
the deepest segments over two workgroups (one of them possibly with no chunks
left), tiles of half identity and half value columns (d_k = d_v) and the
in-order layout otherwise (d_k != d_v, where segment 0 launches no tile of
identity columns only).  The shapes below were chosen with the launch plan's
cost model; the comment of each case says which edge it reaches."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close, oracle_rollout, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call, to_numpy64

pytestmark = pytest.mark.gpu

D64 = WORKLOADS["stream_chunk_h16_d64"]
D128 = WORKLOADS["rollout_h16_d128"]


def _calls(gdn, oracle, wl, calls, *, H, T, null_state=False, api="step", in_place=False,
           out_dtype=torch.float32, what=""):
    announce(f"segments {what}: {wl.name} dk={wl.dk} dv={wl.dv} H={H} T={T} calls={calls} "
             f"null_state={null_state} api={api} in_place={in_place} out={out_dtype}")
    ins = [make_call(wl, c, H=H, T=T) for c in range(calls)]
    if null_state:
        ins[0]["state_in"] = None
    g_outs = []
    state = None
    for c, d in enumerate(ins):
        g = to_dev(d)
        s_in = g["state_in"] if c == 0 else state
        if api == "step":
            kw = dict(out_dtype=out_dtype)
            if in_place and s_in is not None:
                kw["state_out"] = s_in
            o, s = gdn.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], s_in, **kw)
            if in_place and s_in is not None:
                assert s.data_ptr() == s_in.data_ptr()
        else:
            o, s = gdn.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], s_in, wl.chunk,
                                   out_dtype=out_dtype)
        g_outs.append(o.to("cpu", torch.float64).numpy())
        state = s
        if c == 0:
            # later calls carry the state, as the oracle does
            for d2 in ins[1:]:
                d2["state_in"] = None
    torch.cuda.synchronize()
    o_outs, o_state = oracle_rollout(oracle, ins)
    r1 = assert_close(np.concatenate(g_outs, 2), np.concatenate(o_outs, 2), False, what + " out")
    r2 = assert_close(state.to("cpu", torch.float64).numpy(), o_state, False, what + " state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state maxabs {r2[0]:.2e} rel {r2[1]:.2e}",
          flush=True)


def test_d64_last_segment_of_one_chunk(gdn_lib, oracle_mod):
    # 40 chunks: 14 segments of 3, the last of one chunk; segments 11-13 are
    # corrected in halves, so the last segment's second half has no chunk and
    # only applies the map for state_out
    _calls(gdn_lib, oracle_mod, D64, 2, H=16, T=40 * 64, what="d64 last=1")


def test_d64_last_segment_of_one_chunk_null_state_in_place(gdn_lib, oracle_mod):
    _calls(gdn_lib, oracle_mod, D64, 2, H=16, T=40 * 64, null_state=True, in_place=True,
           what="d64 last=1 null state, in place")


def test_d128_eight_segments_ragged(gdn_lib, oracle_mod):
    # 37 chunks: 8 segments of 5 (256 walk workgroups), the last of 2 chunks,
    # which alone is corrected in two halves of one chunk
    _calls(gdn_lib, oracle_mod, D128, 2, H=16, T=37 * 64 - 21, what="d128 8 segments")


def test_d128_eight_segments_bf16_out_null_state(gdn_lib, oracle_mod):
    _calls(gdn_lib, oracle_mod, D128, 1, H=16, T=37 * 64 - 21, null_state=True,
           out_dtype=torch.bfloat16, api="chunked", what="d128 8 segments bf16 out")


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_unequal_head_sizes(gdn_lib, oracle_mod, dk, dv):
    # 8 heads, 42 chunks: 9 segments of 5; tiles in [identity | value] order,
    # segment 0 launches only its tile of value columns; all but one of the
    # corrected segments are split
    _calls(gdn_lib, oracle_mod, D128.replace(dk=dk, dv=dv), 2, H=8, T=2640, what=f"dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_unequal_head_sizes_null_state(gdn_lib, oracle_mod, dk, dv):
    _calls(gdn_lib, oracle_mod, D128.replace(dk=dk, dv=dv), 1, H=8, T=2640, null_state=True,
           what=f"dk={dk} dv={dv} null state")


def test_single_frame_two_segments_every_head(gdn_lib, oracle_mod):
    # the single-frame step's plan: 48 heads, 14 chunks in two segments of 7,
    # segment 0 from the carried state, segment 1 corrected by one workgroup
    _calls(gdn_lib, oracle_mod, WORKLOADS["frame_step_b2_h24_d128"].replace(B=1), 3, H=48, T=880,
           in_place=True, what="single frame, 48 heads")


def test_direct_segment_zero_is_deterministic_and_resumable(gdn_lib):
    # two calls in one equal one call over both halves' tokens only up to
    # rounding, but a repeated call is bit for bit the same, and a state
    # copied to the host after the first call resumes bit for bit
    d = [to_dev(make_call(D128, c, H=16, T=2640)) for c in range(2)]
    announce("segments: determinism and resume, d128 H16")
    o1, s1 = gdn_lib.fwd_step(d[0]["q"], d[0]["k"], d[0]["v"], d[0]["alpha"], d[0]["beta"],
                              d[0]["state_in"])
    o1b, s1b = gdn_lib.fwd_step(d[0]["q"], d[0]["k"], d[0]["v"], d[0]["alpha"], d[0]["beta"],
                                d[0]["state_in"])
    host = s1.cpu()
    o2, s2 = gdn_lib.fwd_step(d[1]["q"], d[1]["k"], d[1]["v"], d[1]["alpha"], d[1]["beta"], s1)
    o2r, s2r = gdn_lib.fwd_step(d[1]["q"], d[1]["k"], d[1]["v"], d[1]["alpha"], d[1]["beta"],
                                host.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o1b) and torch.equal(s1, s1b)
    assert torch.equal(o2, o2r) and torch.equal(s2, s2r)


def _gated(gdn, oracle, wl, calls, *, H, T, chunk=None, out_dtype=torch.float32, what=""):
    announce(f"segments gated {what}: {wl.name} dk={wl.dk} dv={wl.dv} H={H} T={T} calls={calls} "
             f"chunk={chunk} out={out_dtype}")
    g_outs, o_outs = [], []
    g_state = o_state = None
    for c in range(calls):
        d = make_call(wl, c, H=H, T=T, gates=True)
        g = to_dev(d)
        s_in = g["state_in"] if c == 0 else g_state
        kw = dict(out_dtype=out_dtype, gate_logits=True, out_gate=g["out_gate"])
        if chunk is None:
            o, s = gdn.fwd_step(g["q"], g["k"], g["v"], g["alpha_logit"], g["beta_logit"], s_in, **kw)
        else:
            o, s = gdn.fwd_chunked(g["q"], g["k"], g["v"], g["alpha_logit"], g["beta_logit"], s_in,
                                   chunk, **kw)
        g_outs.append(o.to("cpu", torch.float64).numpy())
        g_state = s
        q, k, v, a, b = (to_numpy64(d[n]) for n in ("q", "k", "v", "alpha_logit", "beta_logit"))
        os_in = to_numpy64(d["state_in"]) if (c == 0 and d["state_in"] is not None) else o_state
        oo, o_state = oracle.gdn_fwd(q, k, v, a, b, os_in, gate_logits=True,
                                     out_gate=to_numpy64(d["out_gate"]))
        o_outs.append(oo)
    torch.cuda.synchronize()
    r1 = assert_close(np.concatenate(g_outs, 2), np.concatenate(o_outs, 2), False, what + " out")
    r2 = assert_close(g_state.to("cpu", torch.float64).numpy(), o_state, False, what + " state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state maxabs {r2[0]:.2e} rel {r2[1]:.2e}",
          flush=True)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gated_d64_last_segment_of_one_chunk(gdn_lib, oracle_mod, out_dtype):
    # gated call (logits and an output gate), 40 chunks in 14 segments: gated
    # calls keep the general form (segment 0 from zero, corrected like the
    # others, the gate applied by the correction pass), split halves included
    _gated(gdn_lib, oracle_mod, D64, 2, H=16, T=40 * 64, out_dtype=out_dtype, what="d64")


@pytest.mark.parametrize("chunk", [32, 64])
def test_gated_d128_segments(gdn_lib, oracle_mod, chunk):
    _gated(gdn_lib, oracle_mod, D128, 2, H=16, T=2640, chunk=chunk, what=f"d128 chunk {chunk}")
