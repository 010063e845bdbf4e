"""GPU parity with q and k shared across heads (Hqk q/k heads for H heads,
head h reading q/k head h // (H // Hqk)): forward, prefill stack, decode
step and backward against the fp64 oracle's grouped functions.

Inputs are the seeded per-head draws of the other tests with q and k cut to
their first Hqk heads (k stays unit-norm).  A grouped call must also equal,
bit for bit, the per-head call on q and k repeated over their heads: the
kernels do the same arithmetic on the same operands.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _grouped(inp, Hqk):
    g = dict(inp)
    g["q"] = inp["q"][:, :Hqk].contiguous()
    g["k"] = inp["k"][:, :Hqk].contiguous()
    return g


def _repeat(x, H):
    return x.repeat_interleave(H // x.shape[1], dim=1).contiguous()


def _check(got, ref, dtype, what):
    g = f64(got)
    assert np.all(np.isfinite(g)), what
    e = max(rel_l2(g, ref), per_head_max(g, ref))
    print(f"{what}: rel_l2 {e:.3e}")
    assert e <= TOL[dtype], (what, e)


@pytest.mark.parametrize("Hqk", [1, 2, 3])
@pytest.mark.parametrize("T", [100, 1000])
@pytest.mark.parametrize("chunk", [16, 64])
def test_f32_fwd_grouped(Hqk, T, chunk):
    cfg = synth.FwdConfig("f32_grouped", 2, 6, T, 64, 32, chunk, "f32", 0.05, 7000 + T + Hqk)
    announce(f"fwd grouped f32 H=6 Hqk={Hqk} T={T} chunk={chunk}")
    inp = _grouped(synth.make_fwd_inputs(cfg), Hqk)
    d = to_dev(inp)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=chunk)
    torch.cuda.synchronize()
    _check(out, oracle.fwd_grouped(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"]), "f32", "out")


@pytest.mark.parametrize("Hqk", [1, 2, 4])
@pytest.mark.parametrize("T", [65, 2048, 3000])
def test_bf16_fwd_grouped(Hqk, T):
    """dk 128, dv 64, chunk 64: the specialised walk, whose workgroup order
    puts the heads of one q/k head side by side."""
    cfg = synth.FwdConfig("bf16_grouped", 1, 8, T, 128, 64, 64, "bf16", 0.05, 7100 + T + Hqk)
    announce(f"fwd grouped bf16 H=8 Hqk={Hqk} T={T}")
    inp = _grouped(synth.make_fwd_inputs(cfg), Hqk)
    d = to_dev(inp)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=64)
    rep = ll.fwd(_repeat(d["q"], 8), _repeat(d["k"], 8), d["v"], d["a"], d["lam"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out, rep)
    _check(out, oracle.fwd_grouped(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"]), "bf16", "out")


@pytest.mark.parametrize("dk,dv,chunk", [(32, 16, 32), (64, 128, 32)])
def test_bf16_fwd_grouped_other_walks(dk, dv, chunk):
    cfg = synth.FwdConfig("bf16_grouped_dims", 2, 4, 900, dk, dv, chunk, "bf16", 0.05, 7200 + dk + dv)
    announce(f"fwd grouped bf16 dk={dk} dv={dv} chunk={chunk}")
    inp = _grouped(synth.make_fwd_inputs(cfg), 2)
    d = to_dev(inp)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=chunk)
    torch.cuda.synchronize()
    _check(out, oracle.fwd_grouped(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"]), "bf16", "out")


def test_bf16_fwd_grouped_16k_sampled():
    """The 16K workload (16 heads) with 2 q/k heads: sampled rows against the
    oracle on the repeated q/k."""
    cfg = synth.WORKLOADS["fwd_bf16_T16K"]
    Hqk = 2
    announce(f"fwd grouped {cfg.name} Hqk={Hqk}")
    inp = _grouped(synth.make_fwd_inputs(cfg), Hqk)
    d = to_dev(inp)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk)
    torch.cuda.synchronize()
    rows = synth.sample_rows(cfg.B, cfg.H, cfg.T, cfg.chunk, 8, seed=91)
    ref = oracle.fwd_rows(_repeat(inp["q"], cfg.H), _repeat(inp["k"], cfg.H), inp["v"], inp["a"], inp["lam"], rows)
    got = f64(out).reshape(cfg.B * cfg.H, cfg.T, cfg.dv)
    g = np.stack([got[bh, t] for bh, t in rows])
    e = rel_l2(g, ref)
    print(f"out: rel_l2 {e:.3e} over {len(rows)} rows")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dtype,T", [("f32", 700), ("bf16", 2049)])
def test_prefill_grouped_then_decode(dtype, T):
    dk, dv, chunk = (64, 32, 32) if dtype == "f32" else (128, 64, 64)
    H, Hqk, steps, Lcap = 4, 2, 3, 17
    cfg = synth.FwdConfig("grouped_prefill", 1, H, T + steps, dk, dv, chunk, dtype, 0.05, 7300 + T)
    announce(f"prefill grouped {dtype} H={H} Hqk={Hqk} T={T}")
    full = _grouped(synth.make_fwd_inputs(cfg), Hqk)
    L = synth.num_levels(T)
    p = {n: x[:, :, :T].contiguous() for n, x in full.items()}
    p["lam"] = p["lam"][..., :L].contiguous()
    d = to_dev(p)
    state = torch.full((1, H, Lcap, dk, dv), float("nan"), device="cuda")
    logscale = torch.full((1, H, Lcap), float("nan"), device="cuda")
    out = ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], state, logscale, chunk=chunk)
    torch.cuda.synchronize()
    _check(out, oracle.fwd_grouped(p["q"], p["k"], p["v"], p["a"], p["lam"]), dtype, "prefill out")
    ref, occ = oracle.prefill_stack(_repeat(p["k"], H), p["v"], p["a"], Lcap)
    st, ls = f64(state), f64(logscale)
    for l in range(Lcap):
        if occ[l]:
            got = np.exp(ls[:, :, l])[..., None, None] * st[:, :, l]
            _check(torch.from_numpy(got), ref[:, :, l], dtype, f"slot {l}")
        else:
            assert np.all(np.isnan(st[:, :, l])), f"free slot {l} written"
    # decode tokens T, T+1, ... with the grouped step
    rows = oracle.fwd_grouped(full["q"], full["k"], full["v"], full["a"], full["lam"])
    dfull = to_dev(full)
    Lf = full["lam"].shape[-1]
    for i in range(steps):
        t = T + i
        lam = torch.zeros((1, H, Lcap), device="cuda")
        lam[..., :Lf] = dfull["lam"][:, :, t]
        pos = torch.full((1,), t, dtype=torch.int64, device="cuda")
        o = ll.decode_step(dfull["q"][:, :, t].contiguous(), dfull["k"][:, :, t].contiguous(),
                           dfull["v"][:, :, t].contiguous(), dfull["a"][:, :, t].contiguous(), lam, state,
                           logscale, pos)
        torch.cuda.synchronize()
        _check(o, rows[:, :, t], dtype, f"decode t={t}")


def test_decode_step_grouped_workload():
    """The batched decode workload's shapes with 2 q/k heads for 16 heads,
    against the oracle step on repeated q/k."""
    cfg = synth.WORKLOADS["decode_bf16_S64"]
    announce(f"decode grouped {cfg.name} Hqk=2")
    inp = synth.make_decode_inputs(cfg)
    inp["q"] = inp["q"][:, :2].contiguous()
    inp["k"] = inp["k"][:, :2].contiguous()
    cpu = {n: x.clone() for n, x in inp.items()}
    d = to_dev(inp)
    o = ll.decode_step(d["q"], d["k"], d["v"], d["a"], d["lam"], d["state"], d["logscale"], d["pos"])
    torch.cuda.synchronize()
    H = cfg.H
    ref_o, ref_state, ref_occ = oracle.decode_step(cpu["state"], cpu["logscale"], cpu["pos"],
                                                   _repeat(cpu["q"], H), _repeat(cpu["k"], H), cpu["v"], cpu["a"],
                                                   cpu["lam"])
    e = rel_l2(f64(o), ref_o)
    print(f"o rel_l2 {e:.3e}")
    assert e <= TOL["bf16"]
    st, g = f64(d["state"]), f64(d["logscale"])
    for s, t in enumerate(cpu["pos"].numpy()):
        for l in oracle.occupied(int(t), cfg.Lcap):
            got = np.exp(g[s, :, l])[:, None, None] * st[s, :, l]
            assert rel_l2(got, ref_state[s, :, l]) <= 1e-5


@pytest.mark.parametrize("dtype,T,chunk", [("f32", 300, 32), ("bf16", 1000, 64), ("bf16", 2049, 32)])
def test_bwd_grouped(dtype, T, chunk):
    dk, dv = (64, 32) if dtype == "f32" else (128, 64)
    H, Hqk = 4, 2
    cfg = synth.FwdConfig("grouped_bwd", 1, H, T, dk, dv, chunk, dtype, 0.05, 7400 + T)
    announce(f"bwd grouped {dtype} H={H} Hqk={Hqk} T={T} chunk={chunk}")
    inp = _grouped(synth.make_fwd_inputs(cfg), Hqk)
    rng = np.random.Generator(np.random.PCG64(7401 + T))
    dout = torch.from_numpy(rng.standard_normal((1, H, T, dv)).astype(np.float32))
    if dtype == "bf16":
        dout = dout.to(torch.bfloat16)
    d = to_dev(inp)
    got = ll.bwd(d["q"], d["k"], d["v"], d["a"], d["lam"], dout.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    assert got[0].shape == inp["q"].shape and got[1].shape == inp["k"].shape
    ref = oracle.bwd_grouped(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"], dout)
    for n, g in zip(("dq", "dk", "dv", "da", "dlam"), got):
        _check(g, ref[n], dtype, n)
