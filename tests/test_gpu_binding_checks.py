"""The Python binding's checks of caller-supplied buffers.  The C ABI sees only
addresses, so a wrong-sized or wrongly typed output buffer would be written
out of bounds by the kernels: the binding must refuse it with ValueError
before any launch.  Also: a call on a side stream (its temporary workspace
allocated by the binding) gives the same bits as on the current stream."""
import pytest
import torch

from gpu_helpers import announce, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import (ATTN_WORKLOADS, FRAME_WORKLOADS, WORKLOADS,
                                                             make_attn_call, make_call, make_frame_call)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def step_inputs():
    return to_dev(make_call(WORKLOADS["stream_chunk_h16_d64"], 0, H=2, T=300))


# built lazily, inside the test: collection runs on machines without a GPU
BAD_BUFFERS = {
    "out wrong shape": lambda B, H, T, dk, dv, dev: dict(out=torch.empty(B, H, T + 1, dv, device=dev)),
    "out wrong dtype": lambda B, H, T, dk, dv, dev: dict(out=torch.empty(B, H, T, dv, dtype=torch.float16,
                                                                         device=dev)),
    "out not contiguous": lambda B, H, T, dk, dv, dev: dict(out=torch.empty(B, H, dv, T,
                                                                            device=dev).transpose(2, 3)),
    "out on the host": lambda B, H, T, dk, dv, dev: dict(out=torch.empty(B, H, T, dv)),
    "state_out wrong dtype": lambda B, H, T, dk, dv, dev: dict(state_out=torch.empty(B, H, dk, dv,
                                                                                     dtype=torch.bfloat16,
                                                                                     device=dev)),
    "state_out wrong shape": lambda B, H, T, dk, dv, dev: dict(state_out=torch.empty(B, H, dv, dk + 1,
                                                                                     device=dev)),
}


@pytest.mark.parametrize("case", list(BAD_BUFFERS))
@pytest.mark.parametrize("entry", ["fwd_step", "fwd_chunked", "fwd_bidir"])
def test_forward_entries_refuse_bad_output_buffers(gdn_lib, step_inputs, entry, case):
    g = step_inputs
    kw = BAD_BUFFERS[case](1, 2, 300, 64, 64, "cuda")
    fn = getattr(gdn_lib, entry)
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
    announce(f"binding check {entry} {case}")
    with pytest.raises(ValueError):
        if entry == "fwd_chunked":
            fn(*args, 64, **kw)
        else:
            fn(*args, **kw)


def test_state_in_must_be_fp32(gdn_lib, step_inputs):
    g = step_inputs
    with pytest.raises(ValueError):
        gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"].to(torch.bfloat16))


def test_framewise_refuses_bad_buffers(gdn_lib):
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"]
    g = to_dev(make_frame_call(wl, 0, H=2, F=2, N=100))
    B, H, T, dk, dv = 1, 2, 200, wl.dk, wl.dv
    args = (g["q"], g["k"], g["v"], g["alpha"], g["beta"], 100)
    for kw in (dict(out=torch.empty(B, H, T, dv + 1, device="cuda")),
               dict(state_out=torch.empty(B, H, dk, dv, dtype=torch.float16, device="cuda")),
               dict(z_out=torch.empty(B, H, dk + 1, device="cuda")),
               dict(z_out=torch.empty(B, H, dk, dtype=torch.bfloat16, device="cuda"))):
        with pytest.raises(ValueError):
            gdn_lib.fwd_framewise(*args, **kw)


def test_attention_refuses_bad_output(gdn_lib):
    wl = ATTN_WORKLOADS["attn_chunk_h16_d64"]
    g = {k: v.cuda().contiguous() for k, v in make_attn_call(wl, 0, H=2, Nq=50, n_sink=30, n_win=0,
                                                             n_cur=50).items()}
    args = [g["q"], g["k_sink"], g["v_sink"], g["k_win"], g["v_win"], g["k_cur"], g["v_cur"]]
    with pytest.raises(ValueError):
        gdn_lib.attn_sink_window(*args, out=torch.empty(1, 2, 51, 64, device="cuda"))
    with pytest.raises(ValueError):
        gdn_lib.attn_sink_window(*args, out=torch.empty(1, 2, 50, 64, dtype=torch.int32, device="cuda"))


def test_side_stream_with_temporary_workspace(gdn_lib):
    # the binding allocates the segment workspace itself and keeps it alive
    # for the side stream; results equal the current stream's bit for bit
    g = to_dev(make_call(WORKLOADS["stream_chunk_h16_d64"], 0))
    announce("binding side stream")
    o1, s1 = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o2, s2 = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], stream=side)
    for _ in range(4):     # allocations on the current stream meanwhile
        torch.empty(1 << 22, device="cuda").fill_(1.0)
    side.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
