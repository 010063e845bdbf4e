"""GPU parity of loglinear_fwd against the fp64 oracle.

Inputs come from the seeded generator; the oracle sees the exact device input
values (bf16 inputs are upcast, not re-drawn).  Small workloads are compared
on every output; the 16K and 64K workloads on a seeded row sample plus every
row of the first, a middle and the last chunk, in the same launch
configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _run(inp, chunk, group_log2=-1, workspace=None, out=None):
    d = to_dev(inp)
    o = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=chunk, group_log2=group_log2,
               workspace=workspace, out=out)
    torch.cuda.synchronize()
    return o


def _check_full(inp, got, dtype):
    ref = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"])
    g = f64(got)
    assert np.all(np.isfinite(g))
    e_all, e_head = rel_l2(g, ref), per_head_max(g, ref)
    print(f"rel_l2={e_all:.3e} worst_head={e_head:.3e}")
    assert e_all <= TOL[dtype] and e_head <= TOL[dtype]
    return ref


def test_tiny_f32_workload():
    cfg = synth.WORKLOADS["tiny_f32_T256"]
    announce(cfg.name)
    inp = synth.make_fwd_inputs(cfg)
    got = _run(inp, cfg.chunk)
    _check_full(inp, got, "f32")


@pytest.mark.parametrize("T", [1, 2, 16, 17, 64, 100, 1000])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_f32_ragged_lengths(T, chunk):
    cfg = synth.FwdConfig("f32_ragged", 1, 2, T, 64, 32, chunk, "f32", 0.05, 2000 + T)
    announce(f"f32 T={T} chunk={chunk}")
    inp = synth.make_fwd_inputs(cfg)
    got = _run(inp, chunk)
    _check_full(inp, got, "f32")


@pytest.mark.parametrize("group_log2", [0, 1, 2, 3])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_f32_full_head_dims_every_group_size(chunk, group_log2):
    """dk=128, dv=64 in fp32: the chunk and group algebra at the tight
    tolerance, with a ragged tail (T not a multiple of the chunk)."""
    cfg = synth.FwdConfig("f32_groups", 1, 2, 1500, 128, 64, chunk, "f32", 0.05, 3000 + chunk)
    announce(f"f32 dk128 dv64 T=1500 chunk={chunk} g={group_log2}")
    inp = synth.make_fwd_inputs(cfg)
    got = _run(inp, chunk, group_log2)
    _check_full(inp, got, "f32")


@pytest.mark.parametrize("dk,dv", [(32, 16), (64, 128), (128, 128), (16, 64)])
def test_f32_other_head_dims(dk, dv):
    cfg = synth.FwdConfig("f32_dims", 1, 2, 700, dk, dv, 32, "f32", 0.05, 4000 + dk + dv)
    announce(f"f32 dk={dk} dv={dv}")
    inp = synth.make_fwd_inputs(cfg)
    _check_full(inp, _run(inp, 32), "f32")


@pytest.mark.parametrize("dk,dv", [(32, 16), (64, 32), (128, 128)])
def test_bf16_other_head_dims(dk, dv):
    cfg = synth.FwdConfig("bf16_dims", 2, 2, 900, dk, dv, 64, "bf16", 0.05, 5000 + dk + dv)
    announce(f"bf16 dk={dk} dv={dv}")
    inp = synth.make_fwd_inputs(cfg)
    _check_full(inp, _run(inp, 64), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_supported_head_size(dtype):
    # every (dk, dv) the forward accepts, each chunk size, one ragged length
    dks = (16, 32, 64, 128) if dtype == "f32" else (32, 64, 128)
    for dk in dks:
        for dv in (16, 32, 64, 128):
            for chunk in (16, 32, 64):
                cfg = synth.FwdConfig("dims", 1, 1, 333, dk, dv, chunk, dtype, 0.05, 7000 + dk + dv + chunk)
                announce(f"{dtype} dk={dk} dv={dv} chunk={chunk}")
                inp = synth.make_fwd_inputs(cfg)
                _check_full(inp, _run(inp, chunk), dtype)


def test_bf16_T2K_workload():
    cfg = synth.WORKLOADS["fwd_bf16_T2K"]
    announce(cfg.name)
    inp = synth.make_fwd_inputs(cfg)
    _check_full(inp, _run(inp, cfg.chunk), "bf16")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("group_log2", [0, 2, 3])
def test_bf16_chunk_and_group_invariance(chunk, group_log2):
    cfg = synth.FwdConfig("bf16_inv", 1, 2, 3000, 128, 64, chunk, "bf16", 0.05, 6000)
    announce(f"bf16 invariance chunk={chunk} g={group_log2}")
    inp = synth.make_fwd_inputs(cfg)
    _check_full(inp, _run(inp, chunk, group_log2), "bf16")


def test_single_chunk_needs_no_workspace():
    cfg = synth.FwdConfig("bf16_one_chunk", 2, 3, 64, 128, 64, 64, "bf16", 0.05, 6100)
    announce("single chunk")
    assert ll.fwd_workspace_bytes(2, 3, 64, 128, 64, 64) == 0
    inp = synth.make_fwd_inputs(cfg)
    _check_full(inp, _run(inp, 64), "bf16")


def _sampled(cfg, inp, per_head_rows=256, seed_off=7):
    """Run the forward in the benchmark's launch configuration and compare a
    seeded row sample (plus every row of the first, a middle and the last
    chunk) with the oracle's rows.  Returns (pooled, worst head, worst row)
    relative L2 errors."""
    got = f64(_run(inp, cfg.chunk)).reshape(cfg.B * cfg.H, cfg.T, cfg.dv)
    assert np.all(np.isfinite(got))
    rows = synth.sample_rows(cfg.B, cfg.H, cfg.T, cfg.chunk, per_head_rows, seed=cfg.seed + seed_off)
    ref = oracle.fwd_rows(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"], rows)
    sel = got[rows[:, 0], rows[:, 1]]
    e = rel_l2(sel, ref)
    worst = max(rel_l2(sel[rows[:, 0] == bh], ref[rows[:, 0] == bh]) for bh in range(cfg.B * cfg.H))
    ref_norm = np.linalg.norm(ref, axis=1)
    zero = ref_norm == 0.0
    # rows whose exact value is 0 (no key at any weighted level) must be 0
    assert np.all(sel[zero] == 0.0)
    row_err = np.where(zero, 0.0, np.linalg.norm(sel - ref, axis=1) / np.where(zero, 1.0, ref_norm))
    i = int(np.argmax(row_err))
    print(f"{len(rows)} rows rel_l2={e:.3e} worst_head={worst:.3e} worst_row={row_err[i]:.3e} "
          f"(head {rows[i, 0]}, t={rows[i, 1]}) median_row={np.median(row_err):.3e}")
    return e, worst, float(row_err[i])


# bf16 inputs with float32 accumulation: the products' operands are the exact
# bf16 inputs, so the error comes from rounding the masked scores, the block
# states and the output to bf16 (unit roundoff 2^-9 each, independent across
# terms): a few 1e-3 relative, measured 2.3-2.6e-3 at 16K and 64K.  The
# pooled and per-head errors must stay within 2x of that; every sampled row
# within the bf16 budget.
BF16_LONG_TOL = 5e-3


@pytest.mark.parametrize("name", ["fwd_bf16_T16K", "fwd_bf16_T64K"])
def test_large_workloads_sampled_rows(name):
    cfg = synth.WORKLOADS[name]
    announce(cfg.name)
    inp = synth.make_fwd_inputs(cfg)
    e, worst, worst_row = _sampled(cfg, inp)
    assert e <= TOL["bf16"] and worst <= TOL["bf16"]
    assert e <= BF16_LONG_TOL and worst <= BF16_LONG_TOL
    assert worst_row <= TOL["bf16"]


def test_far_levels_only_64k():
    """The 64K workload with lambda zero on every level below 10 (the chunk's
    own 6 levels and 4 levels of chunk buckets): each row is then the sum of
    its buckets of at least 512 tokens, i.e. exactly the long-range decay
    offsets and the block states of the far levels, checked per row."""
    cfg = synth.WORKLOADS["fwd_bf16_T64K"]
    announce(f"{cfg.name} far levels only")
    inp = synth.make_fwd_inputs(cfg)
    inp["lam"][..., :10] = 0.0
    e, worst, worst_row = _sampled(cfg, inp, seed_off=11)
    assert e <= BF16_LONG_TOL and worst <= BF16_LONG_TOL
    assert worst_row <= TOL["bf16"]


@pytest.mark.parametrize("T", [16384, 65536])
def test_f32_long_decay_sampled_rows(T):
    """float32 at 16K and 64K tokens with the long-context decay scale
    (a = -softplus(x) * 0.01, so far levels carry mass): sampled rows within
    the float32 tolerance, pooled and per head."""
    cfg = synth.FwdConfig(f"f32_long_T{T}", 1, 2, T, 128, 64, 64, "f32", 0.01, 7000 + T % 1000)
    announce(cfg.name)
    inp = synth.make_fwd_inputs(cfg)
    e, worst, worst_row = _sampled(cfg, inp)
    assert e <= TOL["f32"] and worst <= TOL["f32"]


def test_deterministic_and_workspace_contents_ignored():
    cfg = synth.FwdConfig("bf16_det", 1, 4, 4096, 128, 64, 64, "bf16", 0.05, 6200)
    announce("determinism + NaN-poisoned workspace")
    inp = synth.make_fwd_inputs(cfg)
    n = ll.fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(float("nan"))
    o1 = _run(inp, cfg.chunk, workspace=ws.view(torch.uint8)).clone()
    ws.fill_(float("nan"))
    o2 = _run(inp, cfg.chunk, workspace=ws.view(torch.uint8)).clone()
    o3 = _run(inp, cfg.chunk)
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_output_guard_bands_untouched():
    cfg = synth.FwdConfig("bf16_guard", 1, 2, 1000, 128, 64, 64, "bf16", 0.05, 6300)
    announce("guard bands")
    inp = synth.make_fwd_inputs(cfg)
    n = cfg.B * cfg.H * cfg.T * cfg.dv
    pad = 4096
    buf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + n].view(cfg.B, cfg.H, cfg.T, cfg.dv)
    _run(inp, cfg.chunk, out=out)
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)
    _check_full(inp, out, "bf16")


def _exact_bf16_inputs(B, H, T, dk, dv, seed):
    """Inputs on which the bf16 path rounds nothing: a = 0 (every decay is
    exactly 1), q, k, v sparse in {-1, 0, 1}, lambda a power of two per level.
    Scores, masked scores, chunk and block states and the outputs are then
    small multiples of 1/4, exact in bf16 and fp32 (the test checks this of
    the outputs), so any error is an algebra error."""
    rng = np.random.default_rng(seed)
    L = synth.num_levels(T)

    def sparse(shape, density):
        x = rng.integers(-1, 2, size=shape).astype(np.float32)
        return x * (rng.random(shape) < density)

    q = sparse((B, H, T, dk), 0.08)
    k = sparse((B, H, T, dk), 0.08)
    v = sparse((B, H, T, dv), 0.25)
    lam = np.broadcast_to(2.0 ** -(np.arange(L) % 3), (B, H, T, L)).astype(np.float32).copy()
    return {
        "q": torch.from_numpy(q).to(torch.bfloat16),
        "k": torch.from_numpy(k).to(torch.bfloat16),
        "v": torch.from_numpy(v).to(torch.bfloat16),
        "a": torch.zeros((B, H, T), dtype=torch.float32),
        "lam": torch.from_numpy(lam),
    }


@pytest.mark.parametrize("T,chunk,group_log2", [(4096, 64, 3), (4096, 64, 2), (1500, 32, 3), (777, 16, 1),
                                                 (4096, 64, 0)])
def test_bf16_walk_exact_on_exactly_representable_inputs(T, chunk, group_log2):
    """A tight check of the bf16 kernels' chunk, level and stack algebra
    (the 2e-2 bf16 tolerance alone would hide a small misplaced term)."""
    announce(f"bf16 exact-arithmetic T={T} chunk={chunk} g={group_log2}")
    inp = _exact_bf16_inputs(1, 3, T, 128, 64, 8000 + T)
    got = f64(_run(inp, chunk, group_log2))
    ref = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["lam"])
    assert np.array_equal(torch.from_numpy(ref).to(torch.bfloat16).double().numpy(), ref)
    e = rel_l2(got, ref)
    print(f"rel_l2={e:.3e}")
    assert e <= 1e-5


@pytest.mark.parametrize("B,H,T", [(1, 16, 16384), (1, 3, 5000), (2, 8, 2048)])
def test_one_launch_forward_publishes_every_node(B, H, T):
    # White-box check of the one-launch forward's workspace after a run: every
    # group's ready flag is up and no bounded wait gave up.  Layout: bf16
    # nodes [B*H][nG][128*64], fp32 node totals [B*H][nG], int32 flags
    # [B*H][nG], one int32 count of failed waits (each part 256-byte aligned).
    cfg = synth.FwdConfig("nodes", B, H, T, 128, 64, 64, "bf16", 0.05, 600 + T)
    announce(f"one-launch forward flags B={B} H={H} T={T}")
    d = to_dev(synth.make_fwd_inputs(cfg))
    ws = ll.alloc_workspace(B, H, T, 128, 64, 64)
    ws.fill_(0xAB)
    ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=64, workspace=ws)
    torch.cuda.synchronize()
    al = lambda x: (x + 255) // 256 * 256
    BH, nG = B * H, (T + 127) // 128
    off = al(BH * nG * 128 * 64 * 2) + al(BH * nG * 4)
    flags = ws[off:off + BH * nG * 4].view(torch.int32)
    fails = ws[off + al(BH * nG * 4):off + al(BH * nG * 4) + 4].view(torch.int32)
    assert int(fails.item()) == 0
    assert bool((flags == 1).all()), int((flags != 1).sum())


@pytest.mark.parametrize("as_handle", [False, True])
def test_side_stream_workspace_is_not_reused_early(as_handle, monkeypatch):
    """The binding allocates the workspace on torch's current stream and the
    kernels run on another one.  Queue a long matrix product on the side
    stream first, launch the forward behind it, and on the current stream
    immediately allocate a block of the workspace's size: while the side
    stream has not reached the forward's kernels, the allocator must not hand
    out the workspace's block again.  The output is then checked against the
    oracle."""
    cfg = synth.FwdConfig("bf16_side_stream", 1, 4, 4096, 128, 64, 64, "bf16", 0.05, 6300)
    announce(f"side stream (handle={as_handle})")
    inp = synth.make_fwd_inputs(cfg)
    d = to_dev(inp)
    n = ll.fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk)
    assert n > 0
    made = []
    real_empty = torch.empty

    def spy_empty(*args, **kw):
        t = real_empty(*args, **kw)
        made.append(t.data_ptr())
        return t

    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(16):
            big = big @ big * 1e-2
    monkeypatch.setattr(torch, "empty", spy_empty)
    out = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk,
                 stream=side.cuda_stream if as_handle else side)
    monkeypatch.setattr(torch, "empty", real_empty)
    assert len(made) == 2   # the output and the workspace
    junk = torch.empty(n, dtype=torch.uint8, device="cuda")
    reused = junk.data_ptr() in made
    junk.fill_(0xFF)   # all-ones bytes: NaN as float32 / bfloat16
    torch.cuda.synchronize()
    del junk, big
    assert not reused, "the workspace's block was handed out while the side stream still needed it"
    _check_full(inp, out, "bf16")
