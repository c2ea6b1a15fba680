"""C-ABI contract of libgdn that can be checked without a GPU: the library
loads, exports every entry point declared in include/gdn.h, and rejects bad
arguments synchronously (before any HIP call)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_deltanet_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_recurrence_deltanet_amd import build
        build.build(verbose=False)
    return gdn.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(gdn.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert lib.gdn_version() == 3
    assert lib.gdn_strerror(0) == b"ok"
    assert lib.gdn_strerror(-1) == b"invalid argument"
    assert lib.gdn_strerror(-2) == b"unsupported shape or option"
    assert lib.gdn_strerror(-3) == b"HIP error"


def test_default_opts(lib):
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    assert (o.in_dtype, o.out_dtype, o.qk_l2norm) == (gdn.GDN_BF16, gdn.GDN_F32, 1)
    assert o.scale == 1.0 and abs(o.eps - 1e-6) < 1e-12
    assert o.stream is None and o.workspace is None and o.workspace_bytes == 0
    assert o.gate_logits == 0 and o.out_gate is None


def _call(lib, q=16, k=16, v=16, a=16, b=16, sin=None, out=16, sout=None,
          B=1, H=1, T=8, dk=64, dv=64, chunk=64, opts=None):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn_fwd_chunked(P(q), P(k), P(v), P(a), P(b), P(sin), P(out), P(sout),
                               B, H, T, dk, dv, chunk, opts)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), gdn.GDN_ERR_ARG),
    (dict(out=None), gdn.GDN_ERR_ARG),
    (dict(B=0), gdn.GDN_ERR_ARG),
    (dict(H=-1), gdn.GDN_ERR_ARG),
    (dict(T=-1), gdn.GDN_ERR_ARG),
    (dict(dk=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=256), gdn.GDN_ERR_UNSUPPORTED),
    (dict(chunk=16), gdn.GDN_ERR_UNSUPPORTED),
    (dict(chunk=100), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=24), gdn.GDN_ERR_ARG),          # misaligned
    (dict(sin=8), gdn.GDN_ERR_ARG),         # misaligned state
    (dict(a=17), gdn.GDN_ERR_ARG),          # alpha not element aligned
])
def test_argument_errors_are_synchronous(lib, kw, status):
    # every pointer here is a fake address: validation must reject before any use
    assert _call(lib, **kw) == status
    assert len(lib.gdn_last_error()) > 0


def test_bad_dtype_in_opts(lib):
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    o.in_dtype = 7
    assert _call(lib, opts=ctypes.byref(o)) == gdn.GDN_ERR_ARG
    o.in_dtype = gdn.GDN_F32
    o.out_dtype = 9
    assert _call(lib, opts=ctypes.byref(o)) == gdn.GDN_ERR_ARG


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_fp32_chunk_that_does_not_fit_is_rejected(lib, dk):
    # 128 fp32 rows of a chunk do not fit on chip at any head size
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    o.in_dtype = gdn.GDN_F32
    assert _call(lib, dk=dk, chunk=128, opts=ctypes.byref(o)) == gdn.GDN_ERR_UNSUPPORTED


def test_step_validates_too(lib):
    P = ctypes.c_void_p
    assert lib.gdn_fwd_step(None, P(16), P(16), P(16), P(16), None, P(16), None,
                            1, 1, 4, 64, 64, None) == gdn.GDN_ERR_ARG


def test_workspace_query_is_host_only(lib):
    # few heads: the sequence is split into segments, which needs a workspace
    n = lib.gdn_workspace_bytes(1, 16, 2640, 64, 64, 64, None)
    assert n > 0 and n % 4 == 0
    assert lib.gdn_workspace_bytes(1, 16, 2640, 64, 64, 0, None) == n      # step == chunk 64
    # many heads fill the chip unsplit: no workspace
    assert lib.gdn_workspace_bytes(4, 32, 16384, 128, 128, 64, None) == 0
    assert lib.gdn_workspace_bytes(4, 32, 16384, 128, 128, 128, None) == 0
    # invalid shapes
    assert lib.gdn_workspace_bytes(0, 16, 2640, 64, 64, 64, None) == 0
    assert lib.gdn_workspace_bytes(1, 16, 2640, 48, 64, 64, None) == 0


def test_bidir_needs_its_workspace_before_any_launch(lib):
    P = ctypes.c_void_p
    args = (P(16), P(16), P(16), P(16), P(16), None, P(16), None, 1, 2, 100, 64, 64, 0)
    # no workspace: rejected synchronously (the pointers are fake addresses)
    assert lib.gdn_fwd_bidir(*args, None) == gdn.GDN_ERR_ARG
    assert b"gdn_bidir_workspace_bytes" in lib.gdn_last_error()
    # too small a workspace: same
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    o.workspace = P(4096)
    o.workspace_bytes = 2 * 100 * 64 * 4 - 16
    assert lib.gdn_fwd_bidir(*args, ctypes.byref(o)) == gdn.GDN_ERR_ARG
    # the usual argument checks come first
    assert lib.gdn_fwd_bidir(None, *args[1:], None) == gdn.GDN_ERR_ARG


def _pipe_segment_data(bh, T, dk, dv, chunk, nseg):
    # maps, copy of state_in, Phi, partial outputs, working scales
    rows = -(-(-(-T // chunk)) // nseg) * chunk
    return (bh * nseg * dk * dk * 2 + bh * nseg * dk * dv * 4 + bh * dk * dv * 4
            + bh * nseg * rows * dk * 2 + bh * nseg * rows * dv * 2 + bh * (dv // 16) * 4)


def test_bidir_workspace_query(lib):
    # few heads: the fused call, one set of segment data (256-byte aligned)
    # per direction for the segment count planned for both directions' walks
    got = lib.gdn_bidir_workspace_bytes(1, 16, 2640, 64, 64, 0, None)
    fused = {2 * ((_pipe_segment_data(16, 2640, 64, 64, 64, n) + 255) // 256 * 256)
             for n in range(2, 22) if -(-42 // -(-42 // n)) == n}
    assert got in fused
    plane = (1 * 16 * 2640 * 64 * 4 + 255) // 256 * 256
    assert got > plane
    # fp32 inputs (fp32 walker): the fp32 plane (B*H*T*dv*4 rounded to 256)
    # plus the split-sequence data
    f32 = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(f32))
    f32.in_dtype = gdn.GDN_F32
    assert lib.gdn_bidir_workspace_bytes(1, 16, 2640, 64, 64, 64, ctypes.byref(f32)) == \
        plane + lib.gdn_workspace_bytes(1, 16, 2640, 64, 64, 64, ctypes.byref(f32))
    # many heads: unsegmented, the plane alone
    many = (4 * 32 * 16384 * 128 * 4 + 255) // 256 * 256
    assert lib.gdn_bidir_workspace_bytes(4, 32, 16384, 128, 128, 64, None) == many
    assert lib.gdn_bidir_workspace_bytes(1, 16, 0, 64, 64, 0, None) == 0
    assert lib.gdn_bidir_workspace_bytes(1, 16, 2640, 48, 64, 0, None) == 0


def _attn(lib, q=16, ks=16, vs=16, ns=8, kw=16, vw=16, nw=8, kc=16, vc=16, nc=8, out=16,
          B=1, H=1, Nq=8, d=64, scale=0.0, opts=None):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn_attn_sink_window(P(q), P(ks), P(vs), ns, P(kw), P(vw), nw, P(kc), P(vc), nc,
                                    P(out), B, H, Nq, d, scale, opts)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), gdn.GDN_ERR_ARG),
    (dict(out=None), gdn.GDN_ERR_ARG),
    (dict(ns=-1), gdn.GDN_ERR_ARG),
    (dict(Nq=-1), gdn.GDN_ERR_ARG),
    (dict(d=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ns=0, nw=0, nc=0), gdn.GDN_ERR_ARG),          # no key at all
    (dict(kc=None), gdn.GDN_ERR_ARG),                    # non-empty segment without keys
    (dict(vs=24), gdn.GDN_ERR_ARG),                      # misaligned
    (dict(q=8), gdn.GDN_ERR_ARG),
])
def test_attn_argument_errors_are_synchronous(lib, kw, status):
    assert _attn(lib, **kw) == status
    assert len(lib.gdn_last_error()) > 0


def test_attn_empty_segments_and_dtype(lib):
    # an empty segment may pass NULL pointers; a zero-size call launches nothing
    assert _attn(lib, Nq=0, ks=None, vs=None, ns=0) == gdn.GDN_OK
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    o.in_dtype = gdn.GDN_F32
    assert _attn(lib, opts=ctypes.byref(o)) == gdn.GDN_ERR_UNSUPPORTED


def test_attn_workspace_query(lib):
    # few query blocks: the key range splits (2 ranges for 16 heads of 64, 3 for 8 of 128)
    assert lib.gdn_attn_workspace_bytes(1, 16, 2640, 2640, 2640, 2640, 64, None) == 2 * 16 * 2640 * 66 * 4
    assert lib.gdn_attn_workspace_bytes(1, 8, 2640, 2640, 2640, 2640, 128, None) == 3 * 8 * 2640 * 130 * 4
    # enough query blocks, or too few key tiles: no split, no workspace
    assert lib.gdn_attn_workspace_bytes(8, 32, 4096, 2640, 2640, 2640, 64, None) == 0
    assert lib.gdn_attn_workspace_bytes(1, 1, 64, 64, 0, 64, 64, None) == 0
    assert lib.gdn_attn_workspace_bytes(1, 16, 2640, 2640, 2640, 2640, 96, None) == 0


def _frame(lib, q=16, k=16, v=16, a=16, b=16, sin=None, zin=None, out=16, sout=None, zout=None,
           B=1, H=2, F=3, N=100, dk=64, dv=64, chunk=0, ws=None, ws_bytes=0):
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    o = gdn.GdnOpts()
    lib.gdn_default_opts(ctypes.byref(o))
    o.workspace = P(ws)
    o.workspace_bytes = ws_bytes
    return lib.gdn_fwd_framewise(P(q), P(k), P(v), P(a), P(b), P(sin), P(zin), P(out), P(sout), P(zout),
                                 B, H, F, N, dk, dv, chunk, ctypes.byref(o))


@pytest.mark.parametrize("kw,status", [
    (dict(), gdn.GDN_ERR_ARG),                       # no workspace
    (dict(N=0), gdn.GDN_ERR_ARG),
    (dict(F=-1), gdn.GDN_ERR_ARG),
    (dict(dk=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(B=2, H=40000), gdn.GDN_ERR_UNSUPPORTED),   # B*H above the grid's 65535
    (dict(q=None, ws=4096, ws_bytes=1 << 40), gdn.GDN_ERR_ARG),
    (dict(zin=8, ws=4096, ws_bytes=1 << 40), gdn.GDN_ERR_ARG),    # misaligned z_in
    (dict(ws=4096, ws_bytes=1000), gdn.GDN_ERR_ARG),               # workspace too small
])
def test_framewise_argument_errors_are_synchronous(lib, kw, status):
    assert _frame(lib, **kw) == status
    assert len(lib.gdn_last_error()) > 0


def test_framewise_workspace_query(lib):
    # partial frame summaries [B*H][F][nsp][dk][dk + dv + 16] fp32, each frame's
    # M^T as bf16 hi and lo [B*H][F][dv][dk], z_f [B*H][F][dk] fp32
    r = lambda n: (n + 255) // 256 * 256
    for (B, H, F, N, dk, dv, nsp) in ((1, 16, 3, 880, 64, 64, 4), (1, 16, 3, 880, 128, 128, 2),
                                      (2, 24, 1, 880, 128, 128, 2), (1, 1, 2, 100, 64, 128, 1)):
        bhf = B * H * F
        want = r(bhf * nsp * dk * (dk + dv + 16) * 4) + 2 * r(bhf * dv * dk * 2) + r(bhf * dk * 4)
        assert lib.gdn_framewise_workspace_bytes(B, H, F, N, dk, dv, 0, None) == want
    assert lib.gdn_framewise_workspace_bytes(1, 16, 3, 880, 32, 64, 0, None) == 0
    assert lib.gdn_framewise_workspace_bytes(1, 16, 0, 880, 64, 64, 0, None) == 0


# last: it reloads the binding module (the fixture's library keeps the old types)
def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(gdn)
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="libgdn.so not found"):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        importlib.reload(gdn)


def test_debug_flags_follow_the_environment(lib, monkeypatch):
    monkeypatch.delenv("GDN_DEBUG_REVERSE_WORKGROUPS", raising=False)
    assert lib.gdn_debug_flags() == 0
    monkeypatch.setenv("GDN_DEBUG_REVERSE_WORKGROUPS", "1")
    assert lib.gdn_debug_flags() & 1
    monkeypatch.setenv("GDN_DEBUG_REVERSE_WORKGROUPS", "0")
    assert lib.gdn_debug_flags() == 0


def _seg_bytes(B, H, dk, dv, chunk, nseg, seg_chunks):
    """Workspace of a segmented pipelined call: maps (A_s fp16, B_s fp32) of
    every segment, a copy of the state, Phi and the partial outputs (fp16)
    of seg_chunks chunks per segment, and the working scales."""
    bh, rows = B * H, seg_chunks * chunk
    return (bh * nseg * dk * dk * 2 + bh * nseg * dk * dv * 4 + bh * dk * dv * 4
            + bh * nseg * rows * dk * 2 + bh * nseg * rows * dv * 2 + bh * (dv // 16) * 4)


def test_launch_plans_of_the_workloads(lib):
    # The plan's segment counts for the five workloads, read back through the
    # workspace query (a host-only computation): the 16-head rollout (d=128)
    # in 7 segments of 6 chunks, the 16-head streaming chunk (d=64) in 14 of
    # 3, the 48-head single frame in 2 of 7, the 128-head prefill unsplit.
    assert lib.gdn_workspace_bytes(1, 16, 2640, 128, 128, 0, None) == _seg_bytes(1, 16, 128, 128, 64, 7, 6)
    assert lib.gdn_workspace_bytes(1, 16, 2640, 64, 64, 0, None) == _seg_bytes(1, 16, 64, 64, 64, 14, 3)
    assert lib.gdn_workspace_bytes(2, 24, 880, 128, 128, 0, None) == _seg_bytes(2, 24, 128, 128, 64, 2, 7)
    assert lib.gdn_workspace_bytes(4, 32, 16384, 128, 128, 64, None) == 0
    # a gated single-frame call keeps the costlier general form of the
    # correction pass in the estimate, and stays unsplit
    # (the options type of the loaded library: an earlier test reloads the binding)
    o = lib.gdn_workspace_bytes.argtypes[-1]._type_()
    lib.gdn_default_opts(ctypes.byref(o))
    o.gate_logits = 1
    assert lib.gdn_workspace_bytes(2, 24, 880, 128, 128, 0, ctypes.byref(o)) == 0
