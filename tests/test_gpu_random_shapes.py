"""GPU parity of gdn_fwd_chunked on seeded random shapes: batch and head
counts, ragged lengths, every (d_k, d_v) pair, the three chunk sizes, bf16
and fp32 inputs, gates on or off, with or without an incoming state -- each
against the fp64 oracle on the same bits, element by element.  The shapes are
drawn once from a fixed seed, so the set is the same on every run."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close, to_dev
from linear_attention_recurrence_deltanet_amd.inputs import WORKLOADS, make_call, to_numpy64

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        f32 = rng.random() < 0.25
        dk = int(rng.choice([32, 64] if f32 else [32, 64, 128]))
        dv = int(rng.choice([32, 64, 128]))
        chunk = int(rng.choice([32, 64] if f32 else [32, 64, 128]))   # fp32 rows: no 128-token chunk
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 6)), T=int(rng.integers(1, 700)),
                        dk=dk, dv=dv, chunk=chunk, f32=f32, gates=bool(rng.random() < 0.4),
                        state=bool(rng.random() < 0.6), seed=int(rng.integers(0, 1 << 20))))
    return out


CASES = _cases()


@pytest.mark.parametrize("c", CASES, ids=[
    f"B{c['B']}H{c['H']}T{c['T']}k{c['dk']}v{c['dv']}C{c['chunk']}{'f32' if c['f32'] else 'bf16'}"
    f"{'-gates' if c['gates'] else ''}{'-state' if c['state'] else ''}" for c in CASES])
def test_random_shape(gdn_lib, oracle_mod, c):
    base = WORKLOADS["tiny_f32" if c["f32"] else "stream_chunk_h16_d64"]
    wl = base.replace(dk=c["dk"], dv=c["dv"], state_sigma=0.3 if c["state"] else None, seed=c["seed"])
    announce(f"random {c}")
    d = make_call(wl, 0, B=c["B"], H=c["H"], T=c["T"], gates=c["gates"])
    g = to_dev(d)
    a_key, b_key = ("alpha_logit", "beta_logit") if c["gates"] else ("alpha", "beta")
    out, st = gdn_lib.fwd_chunked(g["q"], g["k"], g["v"], g[a_key], g[b_key], g["state_in"], c["chunk"],
                                  gate_logits=c["gates"], out_gate=g["out_gate"] if c["gates"] else None)
    torch.cuda.synchronize()
    ref, rs = oracle_mod.gdn_fwd(*(to_numpy64(d[n]) for n in ("q", "k", "v", a_key, b_key)),
                                 None if d["state_in"] is None else to_numpy64(d["state_in"]),
                                 gate_logits=c["gates"],
                                 out_gate=to_numpy64(d["out_gate"]) if c["gates"] else None)
    r1 = assert_close(out.to("cpu", torch.float64).numpy(), ref, c["f32"], "out")
    r2 = assert_close(st.to("cpu", torch.float64).numpy(), rs, c["f32"], "state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state rel {r2[1]:.2e}", flush=True)


def _side_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [dict(H=int(rng.integers(1, 5)), dk=int(rng.choice([64, 128])), dv=int(rng.choice([64, 128])),
                 chunk=int(rng.choice([32, 64])), gates=bool(rng.random() < 0.5), state=bool(rng.random() < 0.5),
                 T=int(rng.integers(1, 600)), F=int(rng.integers(1, 4)), N=int(rng.integers(1, 300)),
                 seed=int(rng.integers(0, 1 << 20))) for _ in range(n)]


BIDIR = _side_cases(6, 7)
FRAME = _side_cases(6, 11)


@pytest.mark.parametrize("c", BIDIR, ids=[f"H{c['H']}T{c['T']}k{c['dk']}v{c['dv']}C{c['chunk']}"
                                          f"{'-gates' if c['gates'] else ''}{'-state' if c['state'] else ''}"
                                          for c in BIDIR])
def test_random_shape_bidir(gdn_lib, oracle_mod, c):
    wl = WORKLOADS["stream_chunk_h16_d64"].replace(dk=c["dk"], dv=c["dv"], seed=c["seed"],
                                                     state_sigma=0.3 if c["state"] else None)
    announce(f"random bidir {c}")
    d = make_call(wl, 0, H=c["H"], T=c["T"], gates=c["gates"])
    g = to_dev(d)
    a_key, b_key = ("alpha_logit", "beta_logit") if c["gates"] else ("alpha", "beta")
    out, st = gdn_lib.fwd_bidir(g["q"], g["k"], g["v"], g[a_key], g[b_key], g["state_in"], c["chunk"],
                                gate_logits=c["gates"], out_gate=g["out_gate"] if c["gates"] else None)
    torch.cuda.synchronize()
    ref, rs = oracle_mod.gdn_bidir(*(to_numpy64(d[n]) for n in ("q", "k", "v", a_key, b_key)),
                                   None if d["state_in"] is None else to_numpy64(d["state_in"]),
                                   gate_logits=c["gates"],
                                   out_gate=to_numpy64(d["out_gate"]) if c["gates"] else None)
    r1 = assert_close(out.to("cpu", torch.float64).numpy(), ref, False, "out")
    r2 = assert_close(st.to("cpu", torch.float64).numpy(), rs, False, "state")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state rel {r2[1]:.2e}", flush=True)


@pytest.mark.parametrize("c", FRAME, ids=[f"H{c['H']}F{c['F']}N{c['N']}k{c['dk']}v{c['dv']}"
                                          f"{'-logits' if c['gates'] else ''}" for c in FRAME])
def test_random_shape_framewise(gdn_lib, oracle_mod, c):
    from linear_attention_recurrence_deltanet_amd.inputs import FRAME_WORKLOADS, make_frame_call
    wl = FRAME_WORKLOADS["frame_stream_h16_d64"].replace(dk=c["dk"], dv=c["dv"], seed=c["seed"])
    announce(f"random framewise {c}")
    d = make_frame_call(wl, 0, H=c["H"], F=c["F"], N=c["N"])
    g = to_dev(d)
    a_key, b_key = ("alpha_logit", "beta_logit") if c["gates"] else ("alpha", "beta")
    out, st, z = gdn_lib.fwd_framewise(g["q"], g["k"], g["v"], g[a_key], g[b_key], c["N"],
                                       gate_logits=c["gates"], out_gate=g["out_gate"])
    torch.cuda.synchronize()
    q, k, v, a, b = (to_numpy64(d[n]) for n in ("q", "k", "v", a_key, b_key))
    if c["gates"]:
        a, _ = oracle_mod.gates(a, np.zeros_like(a))
        _, b = oracle_mod.gates(np.zeros_like(b), b)
    ref, rs, rz = oracle_mod.gdn_framewise(q, k, v, a, b, c["N"], out_gate=to_numpy64(d["out_gate"]))
    r1 = assert_close(out.to("cpu", torch.float64).numpy(), ref, False, "out")
    r2 = assert_close(st.to("cpu", torch.float64).numpy(), rs, False, "state")
    r3 = assert_close(z.to("cpu", torch.float64).numpy(), rz, False, "z")
    print(f"   out maxabs {r1[0]:.2e} rel {r1[1]:.2e} | state rel {r2[1]:.2e} | z rel {r3[1]:.2e}", flush=True)


def _plan_cases(n=24, seed=31337):
    # the launch plans: few and many heads (segmented and unsegmented walks,
    # one or two 64-column tiles), long and short sequences, the step entry
    # and every chunk, bf16 outputs, and v / state_in at random binary scales
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.choice([1, 2, 3, 8, 16, 24, 40])),
                        T=int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 3000)),
                                          int(rng.integers(3000, 6000))])),
                        dk=int(rng.choice([64, 128])), dv=int(rng.choice([64, 128])),
                        chunk=int(rng.choice([0, 32, 64, 128])), bf16_out=bool(rng.random() < 0.25),
                        scale_exp=int(rng.integers(-12, 11)), state=bool(rng.random() < 0.7),
                        seed=int(rng.integers(0, 1 << 20))))
    return out


PLANS = _plan_cases()


@pytest.mark.parametrize("c", PLANS, ids=[
    f"B{c['B']}H{c['H']}T{c['T']}k{c['dk']}v{c['dv']}C{c['chunk']}s{c['scale_exp']}"
    f"{'-bf16out' if c['bf16_out'] else ''}{'-state' if c['state'] else ''}" for c in PLANS])
def test_random_plan(gdn_lib, oracle_mod, c):
    wl = WORKLOADS["stream_chunk_h16_d64"].replace(dk=c["dk"], dv=c["dv"], seed=c["seed"],
                                                     state_sigma=0.1 if c["state"] else None)
    announce(f"random plan {c}")
    d = make_call(wl, 0, B=c["B"], H=c["H"], T=c["T"])
    s = 2.0 ** c["scale_exp"]
    d["v"] = (d["v"].float() * s).to(d["v"].dtype)
    if d["state_in"] is not None:
        d["state_in"] = d["state_in"] * s
    g = to_dev(d)
    odt = torch.bfloat16 if c["bf16_out"] else torch.float32
    if c["chunk"] == 0:
        out, st = gdn_lib.fwd_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], out_dtype=odt)
    else:
        out, st = gdn_lib.fwd_chunked(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state_in"], c["chunk"],
                                      out_dtype=odt)
    torch.cuda.synchronize()
    ref, rs = oracle_mod.gdn_fwd(*(to_numpy64(d[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                 None if d["state_in"] is None else to_numpy64(d["state_in"]))
    o = out.to("cpu", torch.float64).numpy() / s
    r1 = assert_close(o, ref / s, False, "out")
    r2 = assert_close(st.to("cpu", torch.float64).numpy() / s, rs / s, False, "state")
    print(f"   out maxabs/s {r1[0]:.2e} rel {r1[1]:.2e} | state rel {r2[1]:.2e}", flush=True)
