"""GPU parity of loglinear_bwd against the fp64 oracle's gradients.

The oracle differentiates the forward definition term by term (and is
pinned to finite differences and to autograd on the CPU).  Small and ragged
workloads compare every gradient element; the 16K workload compares a seeded
sample of query rows (dq, dlambda), key rows (dk, dv), and da at sampled
positions from the pairs within 2048 tokens (the rest is bounded by the
decay and checked to be negligible).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")

NAMES = ("dq", "dk", "dv", "da", "dlam")


def _dout(cfg, T, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((cfg.B, cfg.H, T, cfg.dv))
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(torch.bfloat16) if cfg.dtype == "bf16" else t


def _run(inp, dout, chunk):
    d = to_dev(inp)
    g = ll.bwd(d["q"], d["k"], d["v"], d["a"], d["lam"], dout.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    return dict(zip(NAMES, g))


def _check_all(inp, dout, got, dtype):
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"], dout)
    worst = {}
    for n in NAMES:
        g = f64(got[n])
        assert np.all(np.isfinite(g)), n
        r = ref[n]
        e = rel_l2(g, r)
        eh = per_head_max(g, r) if np.linalg.norm(r) > 0 else e
        worst[n] = max(e, eh)
    print("rel_l2 " + " ".join(f"{n}={worst[n]:.2e}" for n in NAMES))
    for n in NAMES:
        assert worst[n] <= TOL[dtype], (n, worst[n])


def _case(cfg, chunk, T=None):
    T = cfg.T if T is None else T
    inp = synth.make_fwd_inputs(cfg, T=T)
    dout = _dout(cfg, T, cfg.seed + 7)
    got = _run(inp, dout, chunk)
    _check_all(inp, dout, got, cfg.dtype)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 256, 1000, 1024])
def test_f32_bwd_lengths(T):
    cfg = synth.FwdConfig("f32_bwd", 1, 2, T, 64, 32, 32, "f32", 0.05, 6000 + T)
    announce(f"bwd f32 T={T} chunk=32")
    _case(cfg, 32)


@pytest.mark.parametrize("dk,dv", [(32, 32), (128, 64), (64, 128), (128, 128)])
def test_f32_bwd_head_dims(dk, dv):
    cfg = synth.FwdConfig("f32_bwd_dims", 1, 2, 700, dk, dv, 32, "f32", 0.05, 6100 + dk + dv)
    announce(f"bwd f32 dk={dk} dv={dv}")
    _case(cfg, 32)


def test_f32_bwd_many_w_pieces():
    """94 chunks of 32: blocks of up to 64 chunks, so the W sums combine up
    to eight pieces."""
    cfg = synth.FwdConfig("f32_bwd_long", 1, 1, 3000, 64, 64, 32, "f32", 0.02, 6200)
    announce("bwd f32 T=3000 chunk=32")
    _case(cfg, 32)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 700, 2048, 2049])
@pytest.mark.parametrize("chunk", [32, 64])
def test_bf16_bwd_lengths(T, chunk):
    cfg = synth.FwdConfig("bf16_bwd", 1, 2, T, 128, 64, chunk, "bf16", 0.05, 6300 + T)
    announce(f"bwd bf16 T={T} chunk={chunk}")
    _case(cfg, chunk)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 128)])
def test_bf16_bwd_head_dims(dk, dv):
    cfg = synth.FwdConfig("bf16_bwd_dims", 2, 2, 900, dk, dv, 64, "bf16", 0.05, 6400 + dk + dv)
    announce(f"bwd bf16 dk={dk} dv={dv}")
    _case(cfg, 64)


@pytest.mark.parametrize("dk,dv,chunk", [(32, 32, 32), (64, 128, 64), (128, 128, 32)])
def test_bf16_bwd_head_dims_deep_tree(dk, dv, chunk):
    # 94 or 47 chunks: groups of 8 chunks form a tree of three or four levels
    # over groups, so the stored left block states of every level (and the
    # nodes inside each group) are read in the product's fragment order for
    # these head dims, not only the first level's
    cfg = synth.FwdConfig("bf16_bwd_deep", 1, 2, 3000, dk, dv, chunk, "bf16", 0.05, 6600 + dk + dv + chunk)
    announce(f"bwd bf16 deep tree dk={dk} dv={dv} chunk={chunk}")
    _case(cfg, chunk)


def test_bf16_bwd_16k_workload_sampled():
    """The 16K forward workload: sampled query and key rows against the
    oracle, and da at sampled positions against its windowed oracle."""
    _sampled(synth.WORKLOADS["fwd_bf16_T16K"])


def test_bf16_bwd_nine_key_levels_sampled():
    """258 chunks of 32: the first chunks' keys are seen from nine chunk
    levels, more than two batches of the key-side levels the chunk kernel
    loads into registers (four per batch)."""
    _sampled(synth.FwdConfig("bf16_bwd_258", 1, 2, 8256, 128, 64, 32, "bf16", 0.05, 6500))


def _sampled(cfg):
    announce(f"bwd {cfg.name} (sampled rows)")
    inp = synth.make_fwd_inputs(cfg)
    dout = _dout(cfg, cfg.T, cfg.seed + 7)
    got = _run(inp, dout, cfg.chunk)
    rows = synth.sample_rows(cfg.B, cfg.H, cfg.T, cfg.chunk, 12, seed=77)
    ref = oracle.bwd_rows(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"], dout, rows, rows)
    BH = cfg.B * cfg.H

    def pick(x):
        x = f64(x).reshape(BH, cfg.T, -1)
        return np.stack([x[bh, t] for bh, t in rows])

    for n in ("dq", "dlam", "dk", "dv"):
        e = rel_l2(pick(got[n]), ref[n])
        print(f"{n}: rel_l2 {e:.3e} over {len(rows)} rows")
        assert e <= TOL[cfg.dtype], (n, e)
    # da at sampled positions from the pairs within W tokens of r; the
    # omitted pairs are at least W apart, so each carries a decay of at most
    # exp(largest sum of W consecutive a's), bounded below
    W = 2048
    rng = np.random.Generator(np.random.PCG64(78))
    drows = np.stack([rng.integers(0, BH, 48), rng.integers(1, cfg.T, 48)], axis=1)
    want = oracle.da_window(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"], dout, drows, W)
    a64 = f64(inp["a"]).reshape(BH, cfg.T)
    csum = np.cumsum(a64, axis=1)
    max_window = float(np.max(csum[:, W:] - csum[:, :-W]))
    qn = np.linalg.norm(f64(inp["q"]), axis=-1).max() * np.linalg.norm(f64(inp["k"]), axis=-1).max()
    dn = np.linalg.norm(f64(dout), axis=-1).max() * np.linalg.norm(f64(inp["v"]), axis=-1).max()
    bound = float(cfg.T) ** 2 * qn * dn * np.exp(max_window)
    print(f"da window {W}: omitted-pair bound {bound:.2e}")
    assert bound < 1e-6 * np.linalg.norm(want)
    got_da = f64(got["da"]).reshape(BH, cfg.T)
    gd = np.array([got_da[bh, r] for bh, r in drows])
    e = rel_l2(gd, want)
    print(f"da: rel_l2 {e:.3e} over {len(drows)} positions")
    assert e <= TOL[cfg.dtype]
    assert np.all(got_da[:, 0] == 0.0)
