"""GPU parity of loglinear_prefill: the forward that also writes the decode
stack of the prompt's last position.

Checks, against the fp64 oracle on the same seeded inputs:
  - every occupied slot, materialised as exp(g) * hat S, against the oracle's
    bucket sums (free slots must stay unwritten: they start as NaN);
  - the prefill's output against the oracle, and bit for bit against the
    plain forward (the same kernels);
  - decode of tokens T, T+1, ... from the written stack against rows T, T+1,
    ... of the oracle forward over the longer sequence.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _prompt(inp, T):
    """The first T tokens of a longer draw, lambda cut to num_levels(T)."""
    L = synth.num_levels(T)
    return {
        "q": inp["q"][:, :, :T].contiguous(),
        "k": inp["k"][:, :, :T].contiguous(),
        "v": inp["v"][:, :, :T].contiguous(),
        "a": inp["a"][:, :, :T].contiguous(),
        "lam": inp["lam"][:, :, :T, :L].contiguous(),
    }


def _prefill(p, chunk, Lcap, group_log2=-1):
    d = to_dev(p)
    B, H, T, dk = p["q"].shape
    dv = p["v"].shape[-1]
    state = torch.full((B, H, Lcap, dk, dv), float("nan"), device="cuda")
    logscale = torch.full((B, H, Lcap), float("nan"), device="cuda")
    out = ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], state, logscale, chunk=chunk,
                     group_log2=group_log2)
    torch.cuda.synchronize()
    return d, out, state, logscale


def _check_stack(p, state, logscale, dtype):
    Lcap = state.shape[2]
    ref, occ = oracle.prefill_stack(p["k"], p["v"], p["a"], Lcap)
    st, ls = f64(state), f64(logscale)
    worst = 0.0
    for l in range(Lcap):
        if occ[l]:
            got = np.exp(ls[:, :, l])[..., None, None] * st[:, :, l]
            assert np.all(np.isfinite(got)), l
            e = max(rel_l2(got, ref[:, :, l]), per_head_max(got, ref[:, :, l]))
            worst = max(worst, e)
            assert e <= TOL[dtype], (l, e)
        else:
            assert np.all(np.isnan(st[:, :, l])) and np.all(np.isnan(ls[:, :, l])), f"free slot {l} written"
    print(f"stack: {int(occ.sum())} slots, worst rel_l2 {worst:.3e}")


def _decode_steps(full, d_state, d_logscale, T, steps, rows_ref, dtype):
    """Decode tokens T .. T+steps-1 from the prefill stack; rows_ref[i] is
    the oracle's row T+i of the forward over the longer sequence."""
    B, H, _, dk = full["q"].shape
    Lcap = d_state.shape[2]
    Lfull = full["lam"].shape[-1]
    dfull = to_dev(full)
    for i in range(steps):
        t = T + i
        lam = torch.zeros((B, H, Lcap), device="cuda")
        lam[..., :Lfull] = dfull["lam"][:, :, t]
        pos = torch.full((B,), t, dtype=torch.int64, device="cuda")
        o = ll.decode_step(dfull["q"][:, :, t].contiguous(), dfull["k"][:, :, t].contiguous(),
                           dfull["v"][:, :, t].contiguous(), dfull["a"][:, :, t].contiguous(), lam.contiguous(),
                           d_state, d_logscale, pos)
        torch.cuda.synchronize()
        got = f64(o)
        e = max(rel_l2(got, rows_ref[i]), per_head_max(got, rows_ref[i]))
        print(f"decode t={t}: rel_l2 {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= TOL[dtype], (t, e)


def _case(cfg, T, chunk, group_log2=-1, steps=3, Lcap=17):
    full = synth.make_fwd_inputs(cfg, T=T + steps)
    p = _prompt(full, T)
    d, out, state, logscale = _prefill(p, chunk, Lcap, group_log2)
    _check_stack(p, state, logscale, cfg.dtype)
    ref_full = oracle.fwd(full["q"], full["k"], full["v"], full["a"], full["lam"])
    got = f64(out)
    e = max(rel_l2(got, ref_full[:, :, :T]), per_head_max(got, ref_full[:, :, :T]))
    assert np.all(np.isfinite(got)) and e <= TOL[cfg.dtype], e
    # the prefill's output is the plain forward's, bit for bit (same kernels)
    ref_out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=chunk, group_log2=group_log2)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    ref_rows = ref_full[:, :, T:T + steps]
    _decode_steps(full, state, logscale, T, steps, [ref_rows[:, :, i] for i in range(steps)], cfg.dtype)


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 64, 100, 1000, 1024, 1025])
@pytest.mark.parametrize("chunk", [16, 64])
def test_f32_prefill_lengths(T, chunk):
    cfg = synth.FwdConfig("f32_prefill", 1, 2, T, 64, 32, chunk, "f32", 0.05, 5000 + T)
    announce(f"prefill f32 T={T} chunk={chunk}")
    _case(cfg, T, chunk)


@pytest.mark.parametrize("group_log2", [0, 1, 2, 3])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_f32_prefill_every_group_size(chunk, group_log2):
    """Buckets of whole groups come from the forward's group states; finer
    ones are summed from the keys of the last group.  Both sides of that
    split at every group size, with a ragged tail."""
    cfg = synth.FwdConfig("f32_prefill_g", 1, 2, 1500, 128, 64, chunk, "f32", 0.05, 5100 + chunk)
    announce(f"prefill f32 dk128 dv64 T=1500 chunk={chunk} g={group_log2}")
    _case(cfg, 1500, chunk, group_log2)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16)])
def test_f32_prefill_head_dims(dk, dv):
    cfg = synth.FwdConfig("f32_prefill_dims", 2, 2, 777, dk, dv, 32, "f32", 0.05, 5200 + dk + dv)
    announce(f"prefill f32 dk={dk} dv={dv}")
    _case(cfg, 777, 32)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 384, 700, 2048, 2049])
@pytest.mark.parametrize("group_log2", [-1, 0, 3])
def test_bf16_prefill(T, group_log2):
    cfg = synth.FwdConfig("bf16_prefill", 1, 4, T, 128, 64, 64, "bf16", 0.05, 5300 + T)
    announce(f"prefill bf16 T={T} g={group_log2}")
    _case(cfg, T, 64, group_log2)


@pytest.mark.parametrize("dk,dv", [(32, 16), (64, 128)])
def test_bf16_prefill_head_dims(dk, dv):
    cfg = synth.FwdConfig("bf16_prefill_dims", 2, 2, 1300, dk, dv, 32, "bf16", 0.05, 5400 + dk + dv)
    announce(f"prefill bf16 dk={dk} dv={dv}")
    _case(cfg, 1300, 32)


def test_bf16_prefill_16k_workload():
    """The 16K forward workload as the prompt (the one-launch forward; its
    Fenwick nodes give the stack's whole-group buckets): every stack slot
    against the oracle, then one decode step."""
    cfg = synth.WORKLOADS["fwd_bf16_T16K"]
    T = cfg.T
    announce(f"prefill {cfg.name}")
    full = synth.make_fwd_inputs(cfg, T=T + 1)
    p = _prompt(full, T)
    d, out, state, logscale = _prefill(p, cfg.chunk, 17)
    _check_stack(p, state, logscale, cfg.dtype)
    rows = np.array([[bh, T] for bh in range(cfg.B * cfg.H)])
    ref = oracle.fwd_rows(full["q"], full["k"], full["v"], full["a"], full["lam"], rows)
    ref = ref.reshape(cfg.B, cfg.H, 1, -1)[:, :, 0]
    _decode_steps(full, state, logscale, T, 1, [ref], cfg.dtype)


def test_prefill_empty_prompt_writes_nothing():
    cfg = synth.FwdConfig("f32_prefill_empty", 1, 2, 4, 32, 16, 16, "f32", 0.05, 5500)
    full = synth.make_fwd_inputs(cfg, T=4)
    p = _prompt(full, 0)
    _, out, state, logscale = _prefill(p, 16, 4)
    assert out.numel() == 0
    assert torch.isnan(state).all() and torch.isnan(logscale).all()


@pytest.mark.parametrize("T,dtype,chunk", [(16, "f32", 16), (1024, "f32", 64), (1024, "bf16", 64),
                                           (64, "bf16", 64)])
def test_prefill_with_the_smallest_lcap_then_decode(T, dtype, chunk):
    """Lcap = 1 + bit_length(T), the smallest the prefill accepts: for a
    power-of-two T the stack of position T-1 fits in one slot less, but the
    decode step at position T needs this one.  Stack, then three decode
    steps, against the oracle."""
    Lcap = synth.num_levels(T + 1)
    dk, dv = (128, 64) if dtype == "bf16" else (64, 32)
    cfg = synth.FwdConfig("min_lcap", 1, 2, T, dk, dv, chunk, dtype, 0.05, 5600 + T)
    announce(f"prefill {dtype} T={T} chunk={chunk} Lcap={Lcap} then decode")
    _case(cfg, T, chunk, Lcap=Lcap)
