"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs of the C code
that executes on the CPU: the C ABI's validation layer (ll_api.cpp) and the
fp64 C oracle (oracle/ll_oracle.c).

Two sanitized builds are made in a temporary directory:
  - ll_api.cpp compiled by hipcc with ASan and UBSan on the host side only
    (each -fsanitize= behind -Xarch_host; the device code is untouched) and
    linked with the library's other, unsanitized objects;
  - the C oracle compiled by gcc with ASan and UBSan.
Each is then loaded in a child pytest process (with its sanitizer runtime
preloaded, since the Python interpreter itself is not instrumented) that runs
the CPU tests exercising it: the ABI's argument checks, and the oracle's pins.
Any sanitizer report aborts the child and fails the test.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "log_linear_attention_amd", "csrc")

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)} failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}")
    return r


def _child_pytest(env_extra, tests):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    return _run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *tests],
                cwd=ROOT, env=env, timeout=900)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from log_linear_attention_amd import build as hip_build

    bdir = os.path.join(os.path.dirname(hip_build.LIB), "_build")
    others = [os.path.join(bdir, s.rsplit(".", 1)[0] + ".o") for s in hip_build.SOURCES if s != "ll_api.cpp"]
    if not all(os.path.exists(o) for o in others):
        hip_build.build(verbose=False)
    san = []
    for s in ("address", "undefined"):
        san += ["-Xarch_host", f"-fsanitize={s}"]
    obj = str(tmp_path / "ll_api_san.o")
    flags = [f for f in hip_build.FLAGS if f != "-O3"]
    _run([HIPCC, *flags, "-O1", "-g", *san, "-Xarch_host", "-fno-omit-frame-pointer", "-x", "hip", "-c",
          os.path.join(CSRC, "ll_api.cpp"), "-o", obj])
    lib = str(tmp_path / "libloglinear_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-shared-libasan", obj, *others, "-o", lib])
    rt = _run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(rt), rt
    r = _child_pytest({"LOGLINEAR_LIB": lib, "LD_PRELOAD": rt}, ["tests/test_abi.py"])
    assert " passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libll_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "ll_oracle.c"), "-o", lib, "-lm"])
    rts = [_run(["gcc", f"-print-file-name={n}"]).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    assert all(os.path.exists(p) for p in rts), rts
    tests = ["tests/test_oracle_pins.py"] + sorted(
        os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
        if not p.endswith("test_oracle_pins.py"))
    r = _child_pytest({"ORACLE_LIB": lib, "LD_PRELOAD": ":".join(rts)}, tests)
    assert " passed" in r.stdout
