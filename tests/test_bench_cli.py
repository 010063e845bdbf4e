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


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path):
    """A counter summary carries the hash of the kernel sources it was taken
    on; bench.py reports its traffic only while the sources still hash to it."""
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "k.hip"
    src.write_text("__global__ void k(float *x) { x[0] = 1.f; }  // a comment\n")
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"# summary\nkernel_source_sha: {bench.source_hash([str(src)])}\n"
                       "traffic_bytes_per_launch: 12345\n")
    assert bench.read_traffic(str(summary), [str(src)]) == 12345.0
    src.write_text("__global__ void k(float *x) { x[0] = 1.f; }  // another comment\n")   # comments do not count
    assert bench.read_traffic(str(summary), [str(src)]) == 12345.0
    src.write_text("__global__ void k(float *x) { x[0] = 2.f; }\n")
    assert bench.read_traffic(str(summary), [str(src)]) is None
    assert bench.read_traffic(str(tmp_path / "absent.txt"), [str(src)]) is None
