"""Benchmark of the Gated DeltaNet forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of the whole forward path (gdn_fwd_step through the C ABI:
norms, decay scan, Gram products, triangular solve, state contractions,
outputs and the carried fp32 state) over one batch of synthetic input that is
already resident in device memory.  Inputs rotate over enough distinct sets
that the working set exceeds the 256 MB last-level cache, so every step reads
its q/k/v from HBM.  Prints ONE JSON line (rank 0).

The default workload is the streaming rollout: successive calls over
streaming chunks of 3 latent frames (B=1, H=16, d_k=d_v=128, T=2640 tokens
per call, chunk 64, bf16 inputs), the fp32 state carried in place from call
to call, fp32 output.  Other workloads: --workload NAME.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix cores, published
LLC_BYTES = 256 << 20           # Infinity Cache
KERNEL_SOURCES = ("linear_attention_recurrence_deltanet_amd/csrc/gdn_pipe.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_fwd.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_fwd_single.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_frame.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_attn.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_noalloc.hip",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_common.h",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_kernels.h",
                  "linear_attention_recurrence_deltanet_amd/csrc/gdn_api.cpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, out_bytes=4, state_in=True, out_gate=False) -> int:
    """Bytes one call must move at minimum: q, k, v, alpha, beta read once,
    o written once, fp32 state read (if given) and written once; with an
    output gate, the gate read once."""
    s_in = 2 if wl.dtype == "bf16" else 4
    tokheads = wl.B * wl.H * wl.T
    b = tokheads * (2 * wl.dk * s_in + wl.dv * s_in + 2 * s_in + wl.dv * out_bytes
                    + (wl.dv * s_in if out_gate else 0))
    st = wl.B * wl.H * wl.dk * wl.dv * 4
    return b + st + (st if state_in else 0)


def framewise_algorithmic_bytes(wl, out_bytes=4) -> int:
    """Frame-wise call: q, k, v, beta and the output gate read once (bf16),
    out written once, alpha once per frame, the fp32 numerator and
    denominator states read and written once."""
    bh, T = wl.B * wl.H, wl.T
    return (bh * T * (2 * wl.dk * 2 + wl.dv * 2 + 2 + wl.dv * 2 + wl.dv * out_bytes)
            + bh * wl.F * 2 + 2 * bh * (wl.dk * wl.dv + wl.dk) * 4)


def algorithmic_flops(wl) -> int:
    """6 d_k d_v per token and head: y = M^T k, the rank-1 update, o = M^T q."""
    return 6 * wl.B * wl.H * wl.T * wl.dk * wl.dv


def read_traffic(kernel_hash: str, workload: str, family: str = "gdn_pipe"):
    """HBM traffic per launch from the committed rocprofv3 counter summary
    (profiles/<family>_<workload>_traffic.md), if it was taken on the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", f"{family}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", txt)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash:
        return None
    return float(m_val.group(1))


def cpu_baseline(wl, budget_s: float, gates: bool = False, bidir: bool = False):
    """The fp64 oracle, as it stands, timed on the host cores on distinct
    input sets of the same workload (same gate mode) until about `budget_s`
    seconds pass."""
    import oracle
    from linear_attention_recurrence_deltanet_amd.inputs import make_call, to_numpy64
    oracle.build(force=False)
    nthreads = os.cpu_count() or 1
    sets = [make_call(wl, i, gates=gates) for i in range(2)]
    names = ("q", "k", "v") + (("alpha_logit", "beta_logit") if gates else ("alpha", "beta"))
    npsets = []
    for d in sets:
        npsets.append([to_numpy64(d[n]) for n in names] +
                      [None if d["state_in"] is None else to_numpy64(d["state_in"]),
                       to_numpy64(d["out_gate"]) if gates else None])
    calls = 0
    t0 = time.perf_counter()
    while True:
        q, k, v, a, b, s, og = npsets[calls % len(npsets)]
        scan = oracle.gdn_bidir if bidir else oracle.gdn_fwd
        scan(q, k, v, a, b, s, nthreads=nthreads, gate_logits=gates, out_gate=og)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tokens = calls * wl.B * wl.T
    cpu_model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tokens / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{calls} full calls of the same workload (B={wl.B} H={wl.H} T={wl.T} "
                      f"dk={wl.dk} dv={wl.dv}{', gates' if gates else ''}"
                      f"{', bidirectional' if bidir else ''}) in {el:.1f} s, fp64 token-by-token, "
                      f"OpenMP over (b, h, 16-column block), CPU: {cpu_model}"}


def bench_attention(args):
    """Sink-and-window softmax attention (gdn_attn_sink_window): one step is one
    call over the workload's chunk; MFMA-bound (4 Nq N d flops per head)."""
    import torch
    from linear_attention_recurrence_deltanet_amd import gdn
    from linear_attention_recurrence_deltanet_amd.inputs import ATTN_WORKLOADS, make_attn_call, to_numpy64

    wl = ATTN_WORKLOADS[args.workload]
    lib = gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    nk = wl.n_sink + wl.n_win + wl.n_cur
    per_set = wl.B * wl.H * (wl.Nq + 2 * nk) * wl.d * 2
    nsets = max(2, min(16, (2 * LLC_BYTES) // max(per_set, 1) + 1))
    sets = [{k: v.to(dev).contiguous() for k, v in make_attn_call(wl, i).items()} for i in range(nsets)]
    out = torch.empty(wl.B, wl.H, wl.Nq, wl.d, dtype=out_dt, device=dev)
    stream = torch.cuda.current_stream()
    ws_bytes = int(lib.gdn_attn_workspace_bytes(wl.B, wl.H, wl.Nq, wl.n_sink, wl.n_win, wl.n_cur, wl.d, None))
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    opts = gdn.make_opts(torch.bfloat16, out_dt, stream=stream, workspace=workspace)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    calls = [(P(g["q"]), P(g["k_sink"]), P(g["v_sink"]), wl.n_sink, P(g["k_win"]), P(g["v_win"]), wl.n_win,
              P(g["k_cur"]), P(g["v_cur"]), wl.n_cur, P(out), wl.B, wl.H, wl.Nq, wl.d, 0.0) for g in sets]
    fn = lambda c: lib.gdn_attn_sink_window(*c, ctypes.byref(opts))
    for i in range(args.warmup):
        if fn(calls[i % nsets]) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    torch.cuda.synchronize()
    K = args.steps
    t0e = torch.cuda.Event(enable_timing=True)
    t1e = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0e.record(stream)
    for i in range(K):
        fn(calls[i % nsets])
    t1e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = max(t0e.elapsed_time(t1e), wall * 1e3) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        fn(calls[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    kern_ms = statistics.mean(per)
    flops = 4 * wl.B * wl.H * wl.Nq * nk * wl.d
    achieved = flops / (kern_ms * 1e-3) / 1e12
    res = {
        "metric": "sink+window softmax attention query tokens/sec (bf16, 1 GPU) + % of MFMA roofline vs oracle",
        "value": wl.B * wl.Nq / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "Nq": wl.Nq, "n_sink": wl.n_sink,
                   "n_win": wl.n_win, "n_cur": wl.n_cur, "d": wl.d, "entry": "gdn_attn_sink_window",
                   "out_dtype": args.out_dtype, "input_sets": nsets, "workspace_bytes": ws_bytes},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "kernel": {"avg_ms": kern_ms, "p50_ms": statistics.median(per),
                   "p99_ms": sorted(per)[min(len(per) - 1, int(0.99 * len(per)))],
                   "algorithmic_flops": flops, "source_hash": kernel_source_hash()},
    }
    if not args.no_cpu:
        import oracle
        d = make_attn_call(wl, 0)
        h = 0
        t0 = time.perf_counter()
        while True:
            sl = lambda x: to_numpy64(x[:, h % wl.H:h % wl.H + 1])
            oracle.attn_sink_window(sl(d["q"]), sl(d["k_sink"]), sl(d["v_sink"]), sl(d["k_win"]),
                                    sl(d["v_win"]), sl(d["k_cur"]), sl(d["v_cur"]))
            h += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": h * wl.Nq / wl.H / el, "unit": "tokens/s",
                               "cores": os.cpu_count() or 1, "kind": "oracle",
                               "sample": f"{h} single heads of {wl.name} (Nq={wl.Nq}, {nk} keys, d={wl.d}) "
                                         f"in {el:.1f} s, fp64 numpy (BLAS threads), scaled to all heads"}
    print(json.dumps(res), flush=True)


def bench_framewise(args):
    """Frame-wise GDN with a normalised readout (gdn_fwd_framewise): one step
    is one call over the workload's frames with both states carried in place.
    The call is three launches (frame summaries, scan over frames, readout);
    the roofline figure is the call's algorithmic bytes over its duration."""
    import torch
    import oracle
    from linear_attention_recurrence_deltanet_amd import gdn
    from linear_attention_recurrence_deltanet_amd.inputs import FRAME_WORKLOADS, make_frame_call, to_numpy64

    wl = FRAME_WORKLOADS[args.workload]
    lib = gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    out_bytes = 4 if args.out_dtype == "f32" else 2
    bh, T = wl.B * wl.H, wl.T
    alg_bytes = framewise_algorithmic_bytes(wl, out_bytes)
    per_set = bh * T * (2 * wl.dk + 2 * wl.dv + 2) * 2
    nsets = max(2, min(64, (2 * LLC_BYTES) // per_set + 1))
    sets = [{k: v.to(dev).contiguous() for k, v in make_frame_call(wl, i).items()} for i in range(nsets)]
    state = torch.zeros(wl.B, wl.H, wl.dk, wl.dv, device=dev)
    z = torch.zeros(wl.B, wl.H, wl.dk, device=dev)
    outs = [torch.empty(wl.B, wl.H, T, wl.dv, dtype=out_dt, device=dev) for _ in range(2)]
    ws_bytes = int(lib.gdn_framewise_workspace_bytes(wl.B, wl.H, wl.F, wl.N, wl.dk, wl.dv, 0, None))
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    calls = []
    for i, g in enumerate(sets):
        o = gdn.make_opts(torch.bfloat16, out_dt, True, 1.0, 1e-6, stream, workspace, out_gate=g["out_gate"])
        calls.append(((P(g["q"]), P(g["k"]), P(g["v"]), P(g["alpha"]), P(g["beta"]), P(state), P(z),
                       P(outs[i % 2]), P(state), P(z), wl.B, wl.H, wl.F, wl.N, wl.dk, wl.dv, 0),
                      ctypes.pointer(o)))
    fn = lambda c: lib.gdn_fwd_framewise(*c[0], c[1])
    for i in range(args.warmup):
        if fn(calls[i % nsets]) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    torch.cuda.synchronize()
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(K):
        fn(calls[i % nsets])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = max(t0.elapsed_time(t1), wall * 1e3) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        fn(calls[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    call_ms = statistics.mean(per)
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    if args.copy_calibration:
        x = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
    res = {
        "metric": "frame-wise GDN (normalised readout) tokens/sec (bf16, 1 GPU) + % of HBM roofline vs oracle",
        "value": wl.B * T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "F": wl.F, "N": wl.N, "T": T,
                   "dk": wl.dk, "dv": wl.dv, "entry": "gdn_fwd_framewise",
                   "out_dtype": args.out_dtype, "state": "fp32 numerator and denominator carried",
                   "input_sets": nsets, "workspace_bytes": ws_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic(kernel_source_hash(), wl.name, "gdn_frame")
                     if args.out_dtype == "f32" else None},
        "kernel": {"avg_ms": call_ms, "p50_ms": statistics.median(per),
                   "p99_ms": sorted(per)[min(len(per) - 1, int(0.99 * len(per)))],
                   "algorithmic_bytes": alg_bytes, "launches_per_call": 3},
    }
    if not args.no_cpu:
        names = ("q", "k", "v", "alpha", "beta", "out_gate")
        cpu_sets = [[to_numpy64(make_frame_call(wl, i)[n]) for n in names] for i in range(2)]
        n = 0
        c0 = time.perf_counter()
        ms = mz = None
        while True:
            q, k, v, a, b, og = cpu_sets[n % 2]
            _, ms, mz = oracle.gdn_framewise(q, k, v, a, b, wl.N, ms, mz, out_gate=og)
            n += 1
            el = time.perf_counter() - c0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": n * wl.B * T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} full calls of the same workload in {el:.1f} s, fp64 loop "
                                         f"over frames vectorised over heads (numpy)"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="rollout_h16_d128")
    ap.add_argument("--chunk", type=int, default=0, help="0: gdn_fwd_step; else gdn_fwd_chunked")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--gates", action="store_true",
                    help="alpha, beta as logits mapped in the kernel, and an output gate")
    ap.add_argument("--bidir", action="store_true",
                    help="gdn_fwd_bidir: forward scan plus backward scan within the call")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; a multi-GPU figure is not part of it "
              "(heads and value columns shard with no communication).",
              file=sys.stderr)
        sys.exit(2)

    from linear_attention_recurrence_deltanet_amd.inputs import ATTN_WORKLOADS, FRAME_WORKLOADS
    if args.workload in ATTN_WORKLOADS:
        return bench_attention(args)
    if args.workload in FRAME_WORKLOADS:
        return bench_framewise(args)

    import torch
    from linear_attention_recurrence_deltanet_amd import gdn
    from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call

    wl = WORKLOADS[args.workload]
    if args.chunk:
        wl = wl.replace(chunk=args.chunk)
    lib = gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    out_bytes = 4 if args.out_dtype == "f32" else 2
    state_given = True
    alg_bytes = algorithmic_bytes(wl, out_bytes, state_given, args.gates)

    # distinct resident input sets so the rotation exceeds 2x the LLC
    per_set = (wl.B * wl.H * wl.T * (2 * wl.dk + wl.dv + 2 + (wl.dv if args.gates else 0))
               * (2 if wl.dtype == "bf16" else 4))
    nsets = max(2, min(64, (2 * LLC_BYTES) // max(per_set, 1) + 1))
    sets = []
    for i in range(nsets):
        d = make_call(wl, i, gates=args.gates)
        g = {k: (None if v is None else v.to(dev).contiguous()) for k, v in d.items()}
        sets.append(g)
    st_shape = (wl.B, wl.H, wl.dk, wl.dv)
    state0 = sets[0]["state_in"] if sets[0]["state_in"] is not None else torch.zeros(st_shape, device=dev)
    state = state0.clone()
    outs = [torch.empty(wl.B, wl.H, wl.T, wl.dv, dtype=out_dt, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream()
    ws_opts = gdn.make_opts(sets[0]["q"].dtype, out_dt)
    if args.bidir:
        ws_bytes = int(lib.gdn_bidir_workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, args.chunk,
                                                     ctypes.byref(ws_opts)))
    else:
        ws_bytes = gdn.workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, args.chunk, ws_opts)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    a_key, b_key = ("alpha_logit", "beta_logit") if args.gates else ("alpha", "beta")
    calls = []
    for i, g in enumerate(sets):
        # per input set: its output gate, when gated
        o = gdn.make_opts(g["q"].dtype, out_dt, True, 1.0, 1e-6, stream, workspace,
                          gate_logits=args.gates, out_gate=g["out_gate"] if args.gates else None)
        a = (P(g["q"]), P(g["k"]), P(g["v"]), P(g[a_key]), P(g[b_key]), P(state),
             P(outs[i % 2]), P(state), wl.B, wl.H, wl.T, wl.dk, wl.dv)
        calls.append((a, ctypes.pointer(o)))
    if args.bidir:
        fn = lambda c: lib.gdn_fwd_bidir(*c[0], args.chunk, c[1])
    elif args.chunk:
        fn = lambda c: lib.gdn_fwd_chunked(*c[0], wl.chunk, c[1])
    else:
        fn = lambda c: lib.gdn_fwd_step(*c[0], c[1])

    for i in range(args.warmup):
        st = fn(calls[i % nsets])
        if st != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    torch.cuda.synchronize()

    # timed region: K steps back to back, events only at its two ends
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        fn(calls[i % nsets])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(total_ms, wall * 1e3) / K

    # per-call durations on the launch stream (roofline, latency percentiles),
    # a separate pass so that its event records do not slow the timed one
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        fn(calls[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    kern_ms = statistics.mean(per)
    p50 = statistics.median(per)
    p99 = sorted(per)[min(len(per) - 1, int(0.99 * len(per)))]
    tokens_per_step = wl.B * wl.T

    # host latency of one call including dispatch (call, then wait for it),
    # and a warm figure: the same input set every call, so it stays cached
    host = []
    for i in range(K):
        h0 = time.perf_counter()
        fn(calls[i % nsets])
        torch.cuda.synchronize()
        host.append((time.perf_counter() - h0) * 1e3)
    host.sort()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(K):
        fn(calls[0])
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / K

    if args.copy_calibration:
        x = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()

    khash = kernel_source_hash()
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "GDN fwd tokens/sec (bf16, 1 GPU) + % of HBM/MFMA roofline vs oracle",
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "dk": wl.dk,
                   "dv": wl.dv, "chunk": wl.chunk, "entry": "gdn_fwd_bidir" if args.bidir
                   else "gdn_fwd_chunked" if args.chunk else "gdn_fwd_step", "out_dtype": args.out_dtype, "state": "fp32 carried",
                   "input_sets": nsets, "workspace_bytes": ws_bytes,
                   "gates": "logits in, output gate" if args.gates else "values in, no output gate",
                   "scan": "bidirectional" if args.bidir else "forward"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if (args.gates and args.bidir) or args.out_dtype != "f32" or args.chunk
                     else read_traffic(khash, wl.name + ("_gates" if args.gates else "_bidir" if args.bidir else ""))},
        "kernel": {"avg_ms": kern_ms, "p50_ms": p50, "p99_ms": p99,
                   "host_p50_ms": host[len(host) // 2], "host_p99_ms": host[min(len(host) - 1, int(0.99 * len(host)))],
                   "warm_ms_per_call": warm_ms,
                   "algorithmic_bytes": alg_bytes, "algorithmic_flops": algorithmic_flops(wl),
                   # algorithmic flops (6 dk dv per token-head) over the call's duration,
                   # against the dense bf16 matrix-core peak: not a counter reading
                   "algorithmic_flops_frac_of_mfma_peak": algorithmic_flops(wl) / (kern_ms * 1e-3)
                   / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                   "source_hash": khash},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, args.gates, args.bidir)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
