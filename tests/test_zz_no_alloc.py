"""loglinear_fwd_noalloc, the forward for callers that cannot allocate, run
through the C ABI against the plain forward (loglinear_fwd with a caller
workspace) on the same seeded inputs.  Both run the same kernels, so their
outputs must agree bit for bit; the smallest case is also checked against
the fp64 oracle.  Each sequence makes two or more calls in a row, the later
ones smaller, so a call must not depend on what an earlier one left in the
library's scratch."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, announce, f64, per_head_max, rel_l2, to_dev

pytestmark = pytest.mark.gpu

ll = pytest.importorskip("log_linear_attention_amd")


def _pair(cfg):
    d = to_dev(synth.make_fwd_inputs(cfg))
    ref = ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk)
    out = torch.full_like(ref, float("nan"))
    ll.fwd_noalloc(d["q"], d["k"], d["v"], d["a"], d["lam"], out, chunk=cfg.chunk)
    torch.cuda.synchronize()
    return d, ref, out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_plain_forward_then_a_smaller_call(dtype):
    dk, dv, chunk = (128, 64, 64) if dtype == "bf16" else (64, 32, 32)
    # large first, then smaller: the headline 16K shape (bf16: the one-launch
    # forward with 32 MB of nodes and flags), then a ragged 1000-token one
    shapes = [(1, 16, 16384), (1, 2, 1000)] if dtype == "bf16" else [(1, 4, 4096), (1, 2, 1000)]
    for i, (B, H, T) in enumerate(shapes):
        cfg = synth.FwdConfig("noalloc", B, H, T, dk, dv, chunk, dtype, 0.05, 9100 + i)
        announce(f"noalloc {dtype} B={B} H={H} T={T} call {i + 1}")
        d, ref, out = _pair(cfg)
        assert torch.equal(out, ref), f"call {i + 1} differs from loglinear_fwd"
        if i == len(shapes) - 1:
            h = {n: x.cpu() for n, x in d.items()}
            want = oracle.fwd(h["q"], h["k"], h["v"], h["a"], h["lam"])
            got = f64(out)
            e = max(rel_l2(got, want), per_head_max(got, want))
            print(f"call {i + 1} vs oracle: rel_l2 {e:.3e}")
            assert np.all(np.isfinite(got)) and e <= TOL[dtype]

