"""GPU parity of the frame-wise scan with a normalised readout
(gdn_fwd_framewise; SANA-Streaming section 2.1, "Frame-wise Gated DeltaNet":
one decay per frame, a write strength per token, a numerator and a
denominator state carried across chunks, an output gate) against the fp64
oracle (oracle.gdn_framewise) on the same bits: the streaming shapes
(summaries split over tokens), many heads, every (d_k, d_v) pair, ragged
frame lengths down to one token, both states carried over calls and updated
in place, gate logits, no output gate, bf16 outputs, a call without
frames."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL_BF16, announce, assert_close, errors, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import FRAME_WORKLOADS, make_frame_call, to_numpy64

pytestmark = pytest.mark.gpu


def _run(gdn, oracle, wl, calls, *, B=None, H=None, F=None, N=None, gate=True, logits=False,
         out_dtype=torch.float32, in_place=False, what=""):
    N = wl.N if N is None else N
    announce(f"framewise {what} {wl.name} calls={calls} B={B or wl.B} H={H or wl.H} F={F or wl.F} N={N} "
             f"gate={gate} logits={logits} out={out_dtype} in_place={in_place}")
    g_outs, o_outs = [], []
    gs = gz = os_ = oz = None
    for c in range(calls):
        d = make_frame_call(wl, c, B=B, H=H, F=F, N=N)
        g = to_dev(d)
        a_key, b_key = ("alpha_logit", "beta_logit") if logits else ("alpha", "beta")
        kw = dict(out_dtype=out_dtype, gate_logits=logits, out_gate=g["out_gate"] if gate else None)
        if in_place and gs is not None:
            kw.update(state_out=gs, z_out=gz)
        o, gs, gz = gdn.fwd_framewise(g["q"], g["k"], g["v"], g[a_key], g[b_key], N, gs, gz, **kw)
        g_outs.append(o.to("cpu", torch.float64).numpy())
        q, k, v, a, b = (to_numpy64(d[n]) for n in ("q", "k", "v", a_key, b_key))
        if logits:
            a, _ = oracle.gates(a, np.zeros_like(a))
            _, b = oracle.gates(np.zeros_like(b), b)
        oo, os_, oz = oracle.gdn_framewise(q, k, v, a, b, N, os_, oz,
                                           out_gate=to_numpy64(d["out_gate"]) if gate else None)
        o_outs.append(oo)
    torch.cuda.synchronize()
    r1 = assert_close(np.concatenate(g_outs, 2), np.concatenate(o_outs, 2), False, what + " out")
    r2 = assert_close(gs.to("cpu", torch.float64).numpy(), os_, False, what + " state")
    r3 = assert_close(gz.to("cpu", torch.float64).numpy(), oz, False, what + " z")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state rel {r2[1]:.2e} | z rel {r3[1]:.2e}",
          flush=True)


def test_framewise_stream_d64(gdn_lib, oracle_mod):
    # 16 heads, 3 frames of 880 tokens: summaries split four ways per frame
    _run(gdn_lib, oracle_mod, FRAME_WORKLOADS["frame_stream_h16_d64"], 1, what="stream")


def test_framewise_rollout_d128_carried_in_place(gdn_lib, oracle_mod):
    # all 16 heads, both states carried over three calls, updated in place (d = 128)
    _run(gdn_lib, oracle_mod, FRAME_WORKLOADS["frame_rollout_h16_d128"], 3, in_place=True,
         what="rollout")


def test_framewise_many_heads(gdn_lib, oracle_mod):
    # 48 heads of 128, one frame per call
    _run(gdn_lib, oracle_mod, FRAME_WORKLOADS["frame_rollout_h16_d128"], 2, B=2, H=24, F=1,
         what="many-heads")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_framewise_mixed_head_sizes(gdn_lib, oracle_mod, dk, dv):
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"].replace(dk=dk, dv=dv)
    _run(gdn_lib, oracle_mod, wl, 2, H=3, F=2, N=300, what=f"dk{dk}-dv{dv}")


@pytest.mark.parametrize("N", [1, 7, 37, 100, 129])
def test_framewise_ragged_frames(gdn_lib, oracle_mod, N):
    # frames that end inside a 32-token step or a 16-token readout block,
    # and one-token frames (the token-wise rule)
    F = max(2, 300 // N) if N > 1 else 64
    _run(gdn_lib, oracle_mod, FRAME_WORKLOADS["frame_stream_h16_d64"], 2, H=2, F=F, N=N,
         what=f"ragged N={N}")


def test_framewise_gate_logits(gdn_lib, oracle_mod):
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"]
    _run(gdn_lib, oracle_mod, wl, 1, H=4, F=2, N=300, logits=True, what="logits")
    _run(gdn_lib, oracle_mod, wl, 2, H=4, F=2, N=300, gate=False, what="no-gate")


def test_framewise_d128_logits(gdn_lib, oracle_mod):
    wl = FRAME_WORKLOADS["frame_rollout_h16_d128"]
    _run(gdn_lib, oracle_mod, wl, 1, H=4, F=3, N=250, logits=True, what="d128-logits")


def test_framewise_bf16_out_is_fp32_out_rounded_once(gdn_lib, oracle_mod):
    """bf16 outputs are the fp32 outputs rounded once (bit for bit) and meet
    the bf16 bar against the oracle (their rel-L2 is the fp32 error plus the
    bf16 rounding of the output itself, about 1.7e-3 of it)."""
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"]
    announce(f"framewise bf16-out {wl.name}")
    d = make_frame_call(wl, 0)
    g = to_dev(d)
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], wl.N)
    o32, s32, z32 = gdn_lib.fwd_framewise(*args, out_gate=g["out_gate"])
    o16, s16, z16 = gdn_lib.fwd_framewise(*args, out_gate=g["out_gate"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 outputs differ from the rounded fp32 outputs"
    assert torch.equal(s16, s32) and torch.equal(z16, z32)
    ref, _, _ = oracle_mod.gdn_framewise(*(to_numpy64(d[n]) for n in ("q", "k", "v", "alpha", "beta")), wl.N,
                                         out_gate=to_numpy64(d["out_gate"]))
    maxabs, rel = errors(o16.to("cpu", torch.float64).numpy(), ref)
    print(f"   bf16 out maxabs {maxabs:.2e} rel {rel:.2e}", flush=True)
    assert maxabs <= TOL_BF16["maxabs"] and rel <= TOL_BF16["rel"]


def test_framewise_no_frames_copies_states(gdn_lib):
    announce("framewise F=0")
    dev = "cuda"
    B, H, dk, dv = 1, 3, 64, 64
    e = torch.empty(B, H, 0, dk, dtype=torch.bfloat16, device=dev)
    ev = torch.empty(B, H, 0, dv, dtype=torch.bfloat16, device=dev)
    s = torch.randn(B, H, dk, dv, device=dev)
    z = torch.rand(B, H, dk, device=dev)
    o, s2, z2 = gdn_lib.fwd_framewise(e, e, ev, torch.empty(B, H, 0, dtype=torch.bfloat16, device=dev),
                                      torch.empty(B, H, 0, dtype=torch.bfloat16, device=dev), 5, s, z)
    torch.cuda.synchronize()
    assert o.shape == (B, H, 0, dv)
    assert torch.equal(s2, s) and torch.equal(z2, z)
