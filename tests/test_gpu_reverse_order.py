"""Workgroup-order independence: with GDN_DEBUG_REVERSE_WORKGROUPS set, every
launch's workgroups take their work items in reverse order of dispatch.  No
workgroup of a launch reads what another one writes or waits for another, so
every output and state must equal the normal run's bit for bit, on every
launch path: the segment walk and its correction pass, the unsegmented walk,
the 128-token single pass, the fp32 walker, the bidirectional call, the three
frame-wise launches and the split attention with its combine."""
import pytest
import torch

from gpu_helpers import announce, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import (ATTN_WORKLOADS, FRAME_WORKLOADS, WORKLOADS,
                                                             make_attn_call, make_call, make_frame_call)

pytestmark = pytest.mark.gpu
ENV = "GDN_DEBUG_REVERSE_WORKGROUPS"


def _both(monkeypatch, fn):
    from linear_attention_recurrence_deltanet_amd import gdn as gdn_lib
    monkeypatch.delenv(ENV, raising=False)
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv(ENV, "1")
    assert gdn_lib.load().gdn_debug_flags() & 1
    b = fn()
    torch.cuda.synchronize()
    monkeypatch.delenv(ENV)
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)


@pytest.mark.parametrize("name,over,api,chunk", [
    ("stream_chunk_h16_d64", {}, "step", None),                       # segment walk + correction
    ("rollout_h16_d128", {}, "step", None),                           # the same at d = 128
    ("frame_step_b2_h24_d128", {}, "step", None),                     # unsegmented walk
    ("stream_chunk_h16_d64", {"H": 4, "T": 700}, "chunked", 128),     # single pass
    ("tiny_f32", {"H": 3}, "chunked", 64),                            # fp32 walker
])
def test_forward_paths(gdn_lib, monkeypatch, name, over, api, chunk):
    wl = WORKLOADS[name]
    g = to_dev(make_call(wl, 0, **over))
    announce(f"reverse order {name} {over} {api} {chunk}")
    if api == "step":
        fn = lambda: gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"])
    else:
        fn = lambda: gdn_lib.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], chunk)
    _both(monkeypatch, fn)


def test_bidirectional(gdn_lib, monkeypatch):
    g = to_dev(make_call(WORKLOADS["stream_chunk_h16_d64"], 0))
    announce("reverse order bidir")
    _both(monkeypatch, lambda: gdn_lib.fwd_bidir(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"]))


def test_framewise(gdn_lib, monkeypatch):
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"]
    g = to_dev(make_frame_call(wl, 0))
    announce("reverse order framewise")
    _both(monkeypatch, lambda: gdn_lib.fwd_framewise(g["q"], g["k"], g["v"], g["alpha"], g["beta"], wl.N,
                                                     out_gate=g["out_gate"]))


def test_attention_split(gdn_lib, monkeypatch):
    wl = ATTN_WORKLOADS["attn_chunk_h8_d128"]
    d = make_attn_call(wl, 0, H=2, Nq=300, n_sink=1000, n_win=500, n_cur=300)
    g = {k: v.cuda().contiguous() for k, v in d.items()}
    announce("reverse order attention")
    args = [g["q"], g["k_sink"], g["v_sink"], g["k_win"], g["v_win"], g["k_cur"], g["v_cur"]]
    _both(monkeypatch, lambda: (gdn_lib.attn_sink_window(*args),))
