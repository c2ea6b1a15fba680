"""GPU parity of the fused gates (SANA-Streaming appendix G.3 names a decay, a
write and an output gate): alpha and beta given as logits and mapped in the
kernel (alpha = exp(-softplus(a)), beta = sigmoid(b)), and an output gate
multiplying the outputs elementwise -- against the fp64 oracle with the same
maps, on the same bits, on every launch path (segment walk plus correction,
unsegmented walk, fp32 walker, 128-token single pass)."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call, to_numpy64

pytestmark = pytest.mark.gpu


def _run(gdn, oracle, wl, calls, *, B=None, H=None, T=None, chunk=None, api="step",
         logits=True, gate=True, out_dtype=torch.float32, workspace=None, what=""):
    announce(f"gates {what} {wl.name} calls={calls} B={B or wl.B} H={H or wl.H} T={T or wl.T} "
             f"chunk={chunk} api={api} logits={logits} gate={gate} out={out_dtype}")
    g_outs, o_outs = [], []
    g_state = o_state = None
    for c in range(calls):
        d = make_call(wl, c, B=B, H=H, T=T, gates=True)
        g = to_dev(d)
        a_key, b_key = ("alpha_logit", "beta_logit") if logits else ("alpha", "beta")
        og = g["out_gate"] if gate else None
        s_in = g["state_in"] if g["state_in"] is not None else g_state
        kw = dict(out_dtype=out_dtype, gate_logits=logits, out_gate=og)
        if workspace is not None:
            kw["workspace"] = workspace
        if api == "step":
            o, s = gdn.fwd_step(g["q"], g["k"], g["v"], g[a_key], g[b_key], s_in, **kw)
        else:
            o, s = gdn.fwd_chunked(g["q"], g["k"], g["v"], g[a_key], g[b_key], s_in, chunk, **kw)
        g_outs.append(o.to("cpu", torch.float64).numpy())
        g_state = s
        q, k, v, a, b = (to_numpy64(d[n]) for n in ("q", "k", "v", a_key, b_key))
        os_in = to_numpy64(d["state_in"]) if d["state_in"] is not None else o_state
        oo, o_state = oracle.gdn_fwd(q, k, v, a, b, os_in, gate_logits=logits,
                                     out_gate=to_numpy64(d["out_gate"]) if gate else None)
        o_outs.append(oo)
    torch.cuda.synchronize()
    f32 = wl.dtype == "f32"
    r1 = assert_close(np.concatenate(g_outs, 2), np.concatenate(o_outs, 2), f32, what + " out")
    r2 = assert_close(g_state.to("cpu", torch.float64).numpy(), o_state, f32, what + " state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state maxabs {r2[0]:.2e} rel {r2[1]:.2e}",
          flush=True)


@pytest.mark.parametrize("logits,gate", [(True, True), (True, False), (False, True)])
def test_gates_stream_segmented(gdn_lib, oracle_mod, logits, gate):
    # 16 heads, 42 chunks: segment walk and correction pass (d = 64)
    _run(gdn_lib, oracle_mod, WORKLOADS["stream_chunk_h16_d64"], 1, logits=logits, gate=gate,
         what="stream")


def test_gates_rollout_segmented_d128(gdn_lib, oracle_mod):
    _run(gdn_lib, oracle_mod, WORKLOADS["rollout_h16_d128"], 3, H=3, what="rollout")


def test_gates_frame_unsegmented(gdn_lib, oracle_mod):
    # 48 heads, 14 chunks: one unsegmented walk per head (d = 128)
    _run(gdn_lib, oracle_mod, WORKLOADS["frame_step_b2_h24_d128"], 2, what="frame")


def test_gates_unsplit_d64_and_bf16_out(gdn_lib, oracle_mod):
    wl = WORKLOADS["stream_chunk_h16_d64"]
    _run(gdn_lib, oracle_mod, wl, 1, H=4, T=700, workspace=False, what="unsplit")
    _run(gdn_lib, oracle_mod, wl, 1, H=4, T=700, out_dtype=torch.bfloat16, what="bf16-out")


@pytest.mark.parametrize("chunk", [32, 128])
def test_gates_other_chunks(gdn_lib, oracle_mod, chunk):
    _run(gdn_lib, oracle_mod, WORKLOADS["stream_chunk_h16_d64"], 1, H=4, T=1000, api="chunked",
         chunk=chunk, what=f"chunk{chunk}")


@pytest.mark.parametrize("chunk", [32, 64])
def test_gates_fp32(gdn_lib, oracle_mod, chunk):
    _run(gdn_lib, oracle_mod, WORKLOADS["tiny_f32"], 1, api="chunked", chunk=chunk, what="fp32")
