"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_algorithmic_counts():
    """The byte and flop models bench.py divides by: the forward's mandatory
    bytes follow the tensor sizes; the shared-q/k forward drops the q/k heads
    not read."""
    sys.path.insert(0, ROOT)
    import bench
    import synth

    cfg = synth.WORKLOADS["fwd_bf16_T16K"]
    nbytes, flops = bench.fwd_algorithmic(cfg)
    T, H, dk, dv, L = cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.L
    assert nbytes == H * T * ((2 * dk + 2 * dv) * 2 + 4 + 4 * L)
    assert flops > 0
    gflops, gbytes = bench.gdn_algorithmic(synth.WORKLOADS["gdn_f32_T16K"])
    assert set(gflops) == {"ll_gdn_chunk", "ll_gdn_tree", "ll_gdn_walk"}
    assert bench.gdn_algorithmic(synth.WORKLOADS["gdn_f32_T16K"], 2)[1] < gbytes
