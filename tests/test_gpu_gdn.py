"""GPU parity of the Log-Linear Gated DeltaNet forward (float32) against the
fp64 oracle in ``oracle/gdn.py`` (the pairwise sum of the definition, pinned
on the CPU to the recurrent level form, to Gated DeltaNet itself at
lambda = 1 and to the Mamba-2 form for orthogonal keys).

Small and ragged workloads compare every output; the 16K workload compares
a seeded sample of rows (every row of the first, a middle and the last
chunk, plus random rows of every head)."""

import numpy as np
import pytest
import torch

import synth
from oracle import gdn
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _run(inp, chunk):
    d = to_dev(inp)
    out = ll.gdn_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"], chunk=chunk)
    torch.cuda.synchronize()
    return out


def _case(cfg, chunk, T=None):
    inp = synth.make_gdn_inputs(cfg, T=T)
    out = _run(inp, chunk)
    ref = gdn.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["lam"])
    got = f64(out)
    assert np.all(np.isfinite(got))
    e = max(rel_l2(got, ref), per_head_max(got, ref))
    print(f"rel_l2 {e:.3e}")
    assert e <= TOL["f32"], e


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 65, 200, 1000])
@pytest.mark.parametrize("chunk", [32, 64])
def test_gdn_lengths(T, chunk):
    cfg = synth.FwdConfig("gdn_len", 1, 2, T, 128, 64, chunk, "f32", 0.05, 9000 + T)
    announce(f"gdn f32 T={T} chunk={chunk}")
    _case(cfg, chunk)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 128), (32, 64)])
def test_gdn_head_dims(dk, dv):
    cfg = synth.FwdConfig("gdn_dims", 2, 2, 700, dk, dv, 32, "f32", 0.05, 9100 + dk + dv)
    announce(f"gdn f32 dk={dk} dv={dv}")
    _case(cfg, 32)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (32, 64)])
def test_gdn_head_dims_chunk64(dk, dv):
    """Chunks of 64: (128, 128) leaves no LDS for a separate pseudo-value
    buffer, so U is formed in registers and written over V."""
    cfg = synth.FwdConfig("gdn_dims64", 1, 2, 500, dk, dv, 64, "f32", 0.05, 9150 + dk + dv)
    announce(f"gdn f32 dk={dk} dv={dv} chunk=64")
    _case(cfg, 64)


@pytest.mark.parametrize("chunk", [32, 64])
def test_gdn_near_duplicate_keys(chunk):
    """Keys close to one direction, beta in [0.9, 1) and strong decay: the
    chunk's triangular systems far from the identity (large k_i.k_j), the
    transitions close to projections."""
    cfg = synth.FwdConfig("gdn_dup", 1, 2, 300, 64, 32, chunk, "f32", 1.0, 9160 + chunk)
    announce(f"gdn f32 near-duplicate keys chunk={chunk}")
    inp = synth.make_gdn_inputs(cfg)
    rng = np.random.Generator(np.random.PCG64(9170 + chunk))
    k = inp["k"].double()
    k = k[:, :, :1] + 0.2 * k
    inp["k"] = (k / k.norm(dim=-1, keepdim=True)).float().contiguous()
    inp["beta"] = torch.from_numpy(rng.uniform(0.9, 1.0, inp["beta"].shape).astype(np.float32))
    out = _run(inp, chunk)
    ref = gdn.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["lam"])
    got = f64(out)
    assert np.all(np.isfinite(got))
    e = max(rel_l2(got, ref), per_head_max(got, ref))
    print(f"rel_l2 {e:.3e}")
    assert e <= TOL["f32"], e


def test_gdn_many_levels():
    """2600 tokens in chunks of 32: 82 chunks, chunk-level buckets up to
    level 7 of the tree, with a ragged tail."""
    cfg = synth.FwdConfig("gdn_long", 1, 1, 2600, 64, 64, 32, "f32", 0.02, 9200)
    announce("gdn f32 T=2600 chunk=32")
    _case(cfg, 32)


def test_gdn_unit_lambda_is_gated_deltanet():
    cfg = synth.FwdConfig("gdn_unit", 1, 2, 300, 64, 32, 32, "f32", 0.05, 9300)
    announce("gdn f32 lambda = 1")
    inp = synth.make_gdn_inputs(cfg)
    inp["lam"] = torch.ones_like(inp["lam"])
    out = _run(inp, 32)
    ref = gdn.gdn_serial(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"])
    e = rel_l2(f64(out), ref)
    print(f"rel_l2 {e:.3e}")
    assert e <= TOL["f32"]


def test_gdn_16k_workload_sampled():
    cfg = synth.WORKLOADS["gdn_f32_T16K"]
    announce(cfg.name)
    inp = synth.make_gdn_inputs(cfg)
    out = _run(inp, cfg.chunk)
    rows = synth.sample_rows(cfg.B, cfg.H, cfg.T, cfg.chunk, 12, seed=93)
    ref = gdn.gdn_fwd_rows(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["lam"], rows)
    got = f64(out).reshape(cfg.B * cfg.H, cfg.T, cfg.dv)
    g = np.stack([got[bh, t] for bh, t in rows])
    assert np.all(np.isfinite(got))
    e = rel_l2(g, ref)
    print(f"rel_l2 {e:.3e} over {len(rows)} rows")
    assert e <= TOL["f32"]


def _to_bf16(inp):
    d = dict(inp)
    for n in ("q", "k", "v"):
        d[n] = inp[n].to(torch.bfloat16).contiguous()
    return d


@pytest.mark.parametrize("T,chunk", [(1, 64), (65, 64), (1000, 32), (2049, 64)])
def test_gdn_bf16_inputs(T, chunk):
    """bf16 q, k, v (float32 arithmetic, bf16 output) against the oracle on
    the same bf16 values."""
    cfg = synth.FwdConfig("gdn_bf16", 1, 2, T, 128, 64, chunk, "bf16", 0.05, 9400 + T)
    announce(f"gdn bf16 T={T} chunk={chunk}")
    inp = _to_bf16(synth.make_gdn_inputs(cfg))
    out = _run(inp, chunk)
    assert out.dtype == torch.bfloat16
    ref = gdn.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["lam"])
    got = f64(out)
    e = max(rel_l2(got, ref), per_head_max(got, ref))
    print(f"rel_l2 {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= TOL["bf16"], e


def test_gdn_bf16_16k_sampled():
    cfg = synth.WORKLOADS["gdn_f32_T16K"]
    announce(f"{cfg.name} with bf16 inputs")
    inp = _to_bf16(synth.make_gdn_inputs(cfg))
    out = _run(inp, cfg.chunk)
    rows = synth.sample_rows(cfg.B, cfg.H, cfg.T, cfg.chunk, 6, seed=94)
    ref = gdn.gdn_fwd_rows(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], inp["lam"], rows)
    got = f64(out).reshape(cfg.B * cfg.H, cfg.T, cfg.dv)
    g = np.stack([got[bh, t] for bh, t in rows])
    e = rel_l2(g, ref)
    print(f"rel_l2 {e:.3e} over {len(rows)} rows")
    assert e <= TOL["bf16"]


def test_gdn_padded_batch_rows_do_not_see_padding():
    """Prompts of different lengths padded to one T: the form is causal, so
    the real rows of each sequence match the oracle on that sequence alone
    and do not change, bit for bit, when the padding changes."""
    T, lens = 700, [700, 333, 64, 1]
    cfg = synth.FwdConfig("gdn_pad", len(lens), 2, T, 64, 32, 32, "f32", 0.05, 9500)
    announce(f"gdn padded batch lens={lens}")
    inp = synth.make_gdn_inputs(cfg)
    junk = synth.make_gdn_inputs(cfg, seed=9501)
    pad1 = {n: x.clone() for n, x in inp.items()}
    pad2 = {n: x.clone() for n, x in inp.items()}
    for b, Tb in enumerate(lens):
        for n in inp:
            pad1[n][b, :, Tb:] = junk[n][b, :, Tb:]
            pad2[n][b, :, Tb:] = 0.0
    out1 = _run(pad1, 32)
    out2 = _run(pad2, 32)
    for b, Tb in enumerate(lens):
        assert torch.equal(out1[b, :, :Tb], out2[b, :, :Tb]), b
        s = {n: x[b:b + 1, :, :Tb].contiguous() for n, x in inp.items()}
        ref = gdn.gdn_fwd(s["q"], s["k"], s["v"], s["a"], s["beta"], s["lam"])
        e = rel_l2(f64(out1[b:b + 1, :, :Tb]), ref)
        print(f"seq {b} (len {Tb}): rel_l2 {e:.3e}")
        assert e <= TOL["f32"]
