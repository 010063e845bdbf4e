"""GPU parity for batches of prompts of different lengths, padded to one
length T (sequence b holds lens[b] real tokens; the rest is padding drawn
from an unrelated seeded set, finite, with a <= 0).

Each sequence is compared with the fp64 oracle on that sequence alone:
  - forward rows t < lens[b] (and bitwise independence from the padding);
  - loglinear_prefill_varlen's stack of position lens[b] - 1, then decode
    of the next tokens at pos = lens[b];
  - backward with dout zero on the padded rows: the real rows' gradients,
    and zero gradients on the padded rows.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _padded(cfg, T, lens, steps=0):
    """(draw, padded): ``draw`` holds T + steps real tokens per sequence;
    ``padded`` is its first T tokens with rows >= lens[b] replaced by another
    seeded draw, lambda cut to num_levels(T)."""
    draw = synth.make_fwd_inputs(cfg, T=T + steps)
    junk = synth.make_fwd_inputs(cfg, T=T + steps, seed=cfg.seed + 99991)
    L = synth.num_levels(T)
    pad = {}
    for n in draw:
        x = draw[n][:, :, :T].clone()
        for b, Tb in enumerate(lens):
            x[b, :, Tb:] = junk[n][b, :, Tb:T]
        pad[n] = x.contiguous()
    pad["lam"] = pad["lam"][..., :L].contiguous()
    return draw, pad


def _seq(inp, b, Tb):
    return {n: x[b:b + 1, :, :Tb].contiguous() for n, x in inp.items()}


def _err(got, ref):
    return rel_l2(got, ref) if np.linalg.norm(ref) > 0 else float(np.abs(got).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_forward(dtype):
    T, lens = 1000, [1000, 613, 64, 1]
    dk, dv, chunk = (64, 32, 32) if dtype == "f32" else (128, 64, 64)
    cfg = synth.FwdConfig("ragged_fwd", len(lens), 2, T, dk, dv, chunk, dtype, 0.05, 8000)
    announce(f"ragged forward {dtype} lens={lens}")
    draw, pad = _padded(cfg, T, lens)
    d = to_dev(pad)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=chunk)
    # other padding, same real tokens: the real rows must not change at all
    _, pad2 = _padded(synth.FwdConfig("ragged_fwd2", len(lens), 2, T, dk, dv, chunk, dtype, 0.05, 8000), T, lens)
    for n in pad2:
        for b, Tb in enumerate(lens):
            pad2[n][b, :, Tb:] = 0.0 if n != "lam" else 1.0
    d2 = to_dev(pad2)
    out2 = ll.fwd(d2["q"], d2["k"], d2["v"], d2["a"], d2["lam"], chunk=chunk)
    torch.cuda.synchronize()
    for b, Tb in enumerate(lens):
        assert torch.equal(out[b, :, :Tb], out2[b, :, :Tb]), b
        s = _seq(pad, b, Tb)
        ref = oracle.fwd(s["q"], s["k"], s["v"], s["a"], s["lam"])
        e = _err(f64(out[b:b + 1, :, :Tb]), ref)
        print(f"seq {b} (len {Tb}): rel_l2 {e:.3e}")
        assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype,T,lens", [
    ("f32", 700, [700, 333, 1, 0, 129]),
    ("bf16", 2049, [2049, 1500, 1024, 65, 0]),
])
def test_ragged_prefill_then_decode(dtype, T, lens):
    dk, dv, chunk = (64, 32, 32) if dtype == "f32" else (128, 64, 64)
    H, Lcap, steps = 2, 17, 2
    cfg = synth.FwdConfig("ragged_prefill", len(lens), H, T, dk, dv, chunk, dtype, 0.05, 8100 + T)
    announce(f"ragged prefill {dtype} T={T} lens={lens}")
    draw, pad = _padded(cfg, T, lens, steps)
    d = to_dev(pad)
    B = len(lens)
    state = torch.full((B, H, Lcap, dk, dv), float("nan"), device="cuda")
    logscale = torch.full((B, H, Lcap), float("nan"), device="cuda")
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], state, logscale, chunk=chunk, lengths=lens_d)
    torch.cuda.synchronize()
    st, ls = f64(state), f64(logscale)
    for b, Tb in enumerate(lens):
        ref, occ = oracle.prefill_stack(draw["k"][b:b + 1, :, :Tb], draw["v"][b:b + 1, :, :Tb],
                                        draw["a"][b:b + 1, :, :Tb], Lcap)
        for l in range(Lcap):
            if occ[l]:
                got = np.exp(ls[b, :, l])[:, None, None] * st[b, :, l]
                e = _err(got, ref[0, :, l])
                assert np.all(np.isfinite(got)) and e <= TOL[dtype], (b, l, e)
            else:
                assert np.all(np.isnan(st[b, :, l])) and np.all(np.isnan(ls[b, :, l])), (b, l)
    # decode the next tokens of every sequence at its own position
    dd = to_dev(draw)
    Lf = draw["lam"].shape[-1]
    for i in range(steps):
        rows = [Tb + i for Tb in lens]
        pick = lambda x: torch.stack([x[b, :, t] for b, t in enumerate(rows)]).contiguous()
        lam = torch.zeros((B, H, Lcap), device="cuda")
        lam[..., :Lf] = pick(dd["lam"])
        pos = torch.tensor(rows, dtype=torch.int64, device="cuda")
        o = ll.decode_step(pick(dd["q"]), pick(dd["k"]), pick(dd["v"]), pick(dd["a"]), lam, state, logscale, pos)
        torch.cuda.synchronize()
        for b, t in enumerate(rows):
            s = _seq(draw, b, t + 1)
            ref = oracle.fwd_rows(s["q"], s["k"], s["v"], s["a"], s["lam"], [[h, t] for h in range(H)])
            e = _err(f64(o[b]), ref)
            print(f"decode seq {b} t={t}: rel_l2 {e:.3e}")
            assert e <= TOL[dtype], (b, t, e)


def test_ragged_prefill_length_out_of_range():
    """A length above the padded T: that sequence's logscale becomes NaN and
    its state is not written; the others are served."""
    T, lens, H, Lcap = 300, [300, 301, 150], 2, 17
    cfg = synth.FwdConfig("ragged_bad", len(lens), H, T, 64, 32, 32, "f32", 0.05, 8200)
    announce(f"ragged prefill out-of-range length lens={lens}")
    draw, pad = _padded(cfg, T, [300, 300, 150])
    d = to_dev(pad)
    state = torch.full((3, H, Lcap, 64, 32), float("nan"), device="cuda")
    logscale = torch.full((3, H, Lcap), 7.0, device="cuda")
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], state, logscale, chunk=32, lengths=lens_d)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(logscale[1])) and torch.all(torch.isnan(state[1]))
    for b in (0, 2):
        occ = oracle.occupied(lens[b] - 1, Lcap)
        assert torch.all(torch.isfinite(logscale[b, :, occ]))


@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("bf16", 64)])
def test_ragged_backward(dtype, chunk):
    T, lens, H = 900, [900, 417, 64, 1], 2
    dk, dv = (64, 32) if dtype == "f32" else (128, 64)
    cfg = synth.FwdConfig("ragged_bwd", len(lens), H, T, dk, dv, chunk, dtype, 0.05, 8300)
    announce(f"ragged backward {dtype} lens={lens}")
    _, pad = _padded(cfg, T, lens)
    rng = np.random.Generator(np.random.PCG64(8301))
    dout = rng.standard_normal((len(lens), H, T, dv))
    for b, Tb in enumerate(lens):
        dout[b, :, Tb:] = 0.0
    dout = torch.from_numpy(dout.astype(np.float32))
    if dtype == "bf16":
        dout = dout.to(torch.bfloat16)
    d = to_dev(pad)
    got = dict(zip(("dq", "dk", "dv", "da", "dlam"),
                   ll.bwd(d["q"], d["k"], d["v"], d["a"], d["lam"], dout.cuda(), chunk=chunk)))
    torch.cuda.synchronize()
    for b, Tb in enumerate(lens):
        s = _seq(pad, b, Tb)
        ref = oracle.bwd(s["q"], s["k"], s["v"], s["a"], s["lam"], dout[b:b + 1, :, :Tb])
        for n, g in got.items():
            x = f64(g[b:b + 1, :, :Tb])
            r = ref[n]
            if n == "dlam":
                x = x[..., :r.shape[-1]]
            e = _err(x, r)
            print(f"seq {b} {n}: rel_l2 {e:.3e}")
            assert e <= TOL[dtype], (b, n, e)
            # padded rows: exactly zero, except da, whose jumping-pair part is a
            # difference of prefix sums that reach the same total by different
            # summation orders (rounding-level leftovers)
            tail = f64(g[b, :, Tb:])
            if tail.size:
                bound = 1e-5 * float(np.abs(r).max()) if n == "da" else 0.0
                assert float(np.abs(tail).max()) <= bound, (b, n, float(np.abs(tail).max()))


def test_ragged_prefill_with_shared_qk_heads():
    """Prompts of different lengths whose heads share one q/k head: each
    sequence's stack against the oracle on that sequence alone, with its k
    repeated over the heads."""
    T, lens, H, Lcap = 500, [500, 250, 1], 4, 17
    cfg = synth.FwdConfig("ragged_grouped", len(lens), H, T, 64, 32, 32, "f32", 0.05, 8400)
    announce(f"ragged prefill, 1 q/k head for {H} heads, lens={lens}")
    draw, pad = _padded(cfg, T, lens)
    for n in ("q", "k"):
        draw[n] = draw[n][:, :1].contiguous()
        pad[n] = pad[n][:, :1].contiguous()
    d = to_dev(pad)
    B = len(lens)
    state = torch.full((B, H, Lcap, 64, 32), float("nan"), device="cuda")
    logscale = torch.full((B, H, Lcap), float("nan"), device="cuda")
    out = ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], state, logscale, chunk=32,
                     lengths=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    st, ls = f64(state), f64(logscale)
    for b, Tb in enumerate(lens):
        kb = draw["k"][b:b + 1, :, :Tb].repeat_interleave(H, dim=1)
        ref, occ = oracle.prefill_stack(kb, draw["v"][b:b + 1, :, :Tb], draw["a"][b:b + 1, :, :Tb], Lcap)
        for l in range(Lcap):
            if occ[l]:
                got = np.exp(ls[b, :, l])[:, None, None] * st[b, :, l]
                e = _err(got, ref[0, :, l])
                assert e <= TOL["f32"], (b, l, e)
        s = _seq(pad, b, Tb)
        ref_o = oracle.fwd_grouped(s["q"], s["k"], s["v"], s["a"], s["lam"])
        e = _err(f64(out[b:b + 1, :, :Tb]), ref_o)
        print(f"seq {b} (len {Tb}): out rel_l2 {e:.3e}")
        assert e <= TOL["f32"]
