"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import sys

import numpy as np
import torch

from linear_attention_recurrence_deltanet_amd.inputs import Workload, make_call, to_numpy64

# Tolerances: bf16 inputs -> max-abs 2e-2 and rel-L2 2e-3 (both, per tensor);
# fp32 inputs -> rel-L2 1e-4.
TOL_BF16 = dict(maxabs=2e-2, rel=2e-3)
TOL_F32 = dict(rel=1e-4)


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def errors(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / den if den > 0 else np.linalg.norm(d)
    return float(np.abs(d).max()) if d.size else 0.0, float(rel)


def assert_close(got, ref, f32: bool, what: str = ""):
    maxabs, rel = errors(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    if f32:
        assert rel <= TOL_F32["rel"], f"{what}: rel-L2 {rel:.3e} > {TOL_F32['rel']}"
    else:
        assert maxabs <= TOL_BF16["maxabs"], f"{what}: max-abs {maxabs:.3e} > {TOL_BF16['maxabs']}"
        assert rel <= TOL_BF16["rel"], f"{what}: rel-L2 {rel:.3e} > {TOL_BF16['rel']}"
    return maxabs, rel


def to_dev(d: dict, device="cuda"):
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in d.items()}


def gpu_rollout(gdn, wl: Workload, calls: int, *, B=None, H=None, T=None, chunk=None,
                api="chunked", out_dtype=torch.float32, inputs=None):
    """Run `calls` successive calls on the GPU with the state carried.
    Returns (list of per-call outputs as CPU fp64 numpy, final state fp64, inputs list)."""
    chunk = wl.chunk if chunk is None else chunk
    outs, ins = [], []
    state = None
    for c in range(calls):
        d = inputs[c] if inputs is not None else make_call(wl, c, B=B, H=H, T=T)
        ins.append(d)
        g = to_dev(d)
        s_in = g["state_in"] if g["state_in"] is not None else state
        if api == "chunked":
            o, s = gdn.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], s_in,
                                   chunk, out_dtype=out_dtype)
        else:
            o, s = gdn.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], s_in,
                                out_dtype=out_dtype)
        outs.append(o)
        state = s
    torch.cuda.synchronize()
    return ([o.to("cpu", torch.float64).numpy() for o in outs],
            state.to("cpu", torch.float64).numpy(), ins)


def oracle_rollout(oracle, ins, heads=None):
    """The oracle on the same inputs (optionally only the (b, h) pairs in
    `heads`), state carried call to call on its own."""
    outs = []
    state = None
    for d in ins:
        sel = lambda t: t if heads is None else t[[b for b, _ in heads], [h for _, h in heads]][None]
        q, k, v, a, be = (to_numpy64(sel(d[n])) for n in ("q", "k", "v", "alpha", "beta"))
        s0 = d["state_in"]
        s_in = to_numpy64(sel(s0)) if s0 is not None else state
        o, s = oracle.gdn_fwd(q, k, v, a, be, s_in)
        outs.append(o)
        state = s
    return outs, state


def select_heads(arr: np.ndarray, heads):
    return arr[[b for b, _ in heads], [h for _, h in heads]][None]
