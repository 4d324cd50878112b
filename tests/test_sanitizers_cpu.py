"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU oracle and
of the C ABI's host layer (the argument checks, workspace layouts and call
sequences in abi.hip, with stand-in kernel launchers), run on the host.
The HIP sources are built for gfx950 as usual, with each -fsanitize flag
behind -Xarch_host, so only host code is instrumented; nothing runs on a
GPU (the launchers are stand-ins)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
          "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c"),
          "-o", str(exe), "-lm"])
    r = _run([str(exe)], env=dict(ENV, OMP_NUM_THREADS="2"))
    assert r.stdout.startswith("ok")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "mixture_experts_sparse_router_amd", "csrc")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(ROOT, "mixture_experts_sparse_router_amd", "csrc", "abi.hip"),
                os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-x", "hip", "-O1", "-g", "-std=c++17", *inc, *san,
              "-c", src, "-o", str(obj)])
        objs.append(str(obj))
    exe = tmp_path / "abi_san"
    _run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", str(exe)])
    r = _run([str(exe)], env=ENV)
    assert r.stdout.startswith("ok"), r.stdout
