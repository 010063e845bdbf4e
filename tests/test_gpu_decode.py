"""GPU parity of loglinear_decode_step against the fp64 decode oracle, and
consistency of the decode recurrence with the forward."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _materialise(state, logscale, pos, Lcap):
    """True states exp(g) * hat S on the occupied slots of each sequence's
    new position; zeros elsewhere.  Returns (fp64 array, occupancy mask)."""
    st, g = f64(state), f64(logscale)
    out = np.zeros_like(st)
    occ = np.zeros((st.shape[0], Lcap), dtype=bool)
    for s, t in enumerate(np.asarray(pos)):
        if t < 0 or t >= (1 << (Lcap - 1)):
            continue
        for l in oracle.occupied(int(t), Lcap):
            occ[s, l] = True
            out[s, :, l] = np.exp(g[s, :, l])[:, None, None] * st[s, :, l]
    return out, occ


def _step(d):
    o = ll.decode_step(d["q"], d["k"], d["v"], d["a"], d["lam"], d["state"], d["logscale"], d["pos"])
    torch.cuda.synchronize()
    return o


def _check_step(inp, dtype, o_tol=None):
    o_tol = TOL[dtype] if o_tol is None else o_tol
    cpu = {k: v.clone() for k, v in inp.items()}
    d = to_dev(inp)
    o = _step(d)
    ref_o, ref_state, ref_occ = oracle.decode_step(cpu["state"], cpu["logscale"], cpu["pos"], cpu["q"], cpu["k"],
                                                   cpu["v"], cpu["a"], cpu["lam"])
    Lcap = inp["state"].shape[2]
    got_state, occ = _materialise(d["state"], d["logscale"], cpu["pos"].numpy(), Lcap)
    assert np.array_equal(occ, ref_occ)
    e_o = rel_l2(f64(o), ref_o)
    e_s = rel_l2(got_state, ref_state)
    print(f"o rel_l2={e_o:.3e} state rel_l2={e_s:.3e}")
    assert e_o <= o_tol
    assert e_s <= 1e-5
    return o, d


def test_batched_decode_workload():
    cfg = synth.WORKLOADS["decode_bf16_S64"]
    announce(cfg.name)
    _check_step(synth.make_decode_inputs(cfg), "bf16")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128), (32, 64)])
def test_decode_f32_shapes(dk, dv):
    cfg = synth.DecodeConfig("dec_f32", 8, 3, dk, dv, 12, 2000, "f32", 0.05, 7000 + dk + dv)
    announce(f"decode f32 dk={dk} dv={dv}")
    _check_step(synth.make_decode_inputs(cfg), "f32")


def test_decode_position_edge_cases():
    """pos = 0 (empty stack), 1, powers of two (deep merges), 2^(Lcap-1)-1 (all
    levels occupied) and out-of-range positions (NaN, stack untouched)."""
    Lcap = 8
    positions = [0, 1, 2, 3, 4, 64, 127, 128, 129, 255, -1]
    cfg = synth.DecodeConfig("dec_edges", len(positions), 2, 64, 64, Lcap, 100, "f32", 0.05, 7100)
    announce("decode edge positions")
    inp = synth.make_decode_inputs(cfg, positions=positions)
    before = inp["state"].clone()
    before_g = inp["logscale"].clone()
    d = to_dev(inp)
    o = _step(d)
    pos = np.array(positions)
    bad = (pos < 0) | (pos >= (1 << (Lcap - 1)))
    of = f64(o)
    assert np.all(np.isnan(of[bad])) and np.all(np.isfinite(of[~bad]))
    assert torch.equal(d["state"].cpu()[bad], before[bad])
    assert torch.equal(d["logscale"].cpu()[bad], before_g[bad])
    good = np.nonzero(~bad)[0]
    sub = {k: (v[good] if k != "pos" else v[good]) for k, v in inp.items()}
    ref_o, _, _ = oracle.decode_step(sub["state"], sub["logscale"], sub["pos"], sub["q"], sub["k"], sub["v"],
                                     sub["a"], sub["lam"])
    assert rel_l2(of[good], ref_o) <= TOL["f32"]


def test_unoccupied_slots_are_never_read():
    cfg = synth.WORKLOADS["decode_bf16_S64"]
    announce("decode NaN-poisoned free slots")
    inp = synth.make_decode_inputs(cfg)
    poisoned = inp["state"].clone()
    for s, t in enumerate(inp["pos"].tolist()):
        occ = set(oracle.occupied(t - 1, cfg.Lcap))
        for l in range(cfg.Lcap):
            if l not in occ:
                poisoned[s, :, l] = float("nan")
    d1 = to_dev(inp)
    o1 = _step(d1)
    d2 = to_dev(dict(inp, state=poisoned))
    o2 = _step(d2)
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o1, o2)


def test_decode_from_empty_matches_forward():
    """Feeding a sequence token by token through decode_step from an empty
    stack reproduces the forward's rows."""
    B, H, T, dk, dv = 1, 3, 300, 32, 32
    Lcap = synth.num_levels(T)
    cfg = synth.FwdConfig("dec_vs_fwd", B, H, T, dk, dv, 32, "f32", 0.05, 7200)
    announce("decode from empty vs forward")
    inp = synth.make_fwd_inputs(cfg)
    d = to_dev(inp)
    fwd = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=32)
    state = torch.zeros((B, H, Lcap, dk, dv), dtype=torch.float32, device="cuda")
    logscale = torch.zeros((B, H, Lcap), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        o = ll.decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(), d["v"][:, :, t].contiguous(),
                           d["a"][:, :, t].contiguous(), d["lam"][:, :, t].contiguous(), state, logscale, pos)
        outs.append(o.clone())
    torch.cuda.synchronize()
    dec = torch.stack(outs, dim=2)
    ref = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"])
    assert rel_l2(f64(dec), ref) <= TOL["f32"]
    assert rel_l2(f64(dec), f64(fwd)) <= TOL["f32"]


def test_snapshot_and_resume_is_bitwise_identical():
    B, H, T, dk, dv = 2, 2, 80, 64, 64
    Lcap = 8
    cfg = synth.FwdConfig("dec_resume", B, H, T, dk, dv, 16, "bf16", 0.05, 7300)
    announce("decode snapshot/resume")
    d = to_dev(synth.make_fwd_inputs(cfg))
    lam = torch.zeros((B, H, T, Lcap), dtype=torch.float32, device="cuda")
    lam[..., :d["lam"].shape[-1]] = d["lam"]

    def run(state, logscale, t_from, t_to):
        outs = []
        for t in range(t_from, t_to):
            pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
            outs.append(ll.decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                                       d["v"][:, :, t].contiguous(), d["a"][:, :, t].contiguous(),
                                       lam[:, :, t].contiguous(), state, logscale, pos).clone())
        return outs

    s1 = torch.zeros((B, H, Lcap, dk, dv), dtype=torch.float32, device="cuda")
    g1 = torch.zeros((B, H, Lcap), dtype=torch.float32, device="cuda")
    full = run(s1, g1, 0, T)
    s2 = torch.zeros_like(s1)
    g2 = torch.zeros_like(g1)
    run(s2, g2, 0, 37)
    snap_s, snap_g = s2.clone().cpu(), g2.clone().cpu()
    s3, g3 = snap_s.cuda(), snap_g.cuda()
    rest = run(s3, g3, 37, T)
    torch.cuda.synchronize()
    for a, b in zip(full[37:], rest):
        assert torch.equal(a, b)
    assert torch.equal(s1, s3) and torch.equal(g1, g3)
