"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle: oracle.c with a driver that calls every function on small
  seeded inputs (ragged tails, batches, windows, binary16 caches, a decode
  loop past a ring cache's capacity), built with gcc.
* The C ABI: the library sources with the host pass instrumented
  (device code is compiled unoptimised and never run) and a driver that calls
  every entry point with arguments host validation must reject, and with
  valid ones that reach the HIP runtime; on a machine without a GPU those
  return Q4_ERR_HIP.

A sanitizer report aborts the driver, which fails the test.
"""
import os
import shlex
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side instrumentation only: every sanitizer flag goes to the host pass
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
           "-Xarch_host -fno-sanitize-recover=all"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


def _gcc_sanitizers_work(tmp):
    src = os.path.join(tmp, "probe.c")
    with open(src, "w") as f:
        f.write("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", src, "-o", os.path.join(tmp, "probe")],
                       capture_output=True)
    return r.returncode == 0


def test_oracle_under_sanitizers(tmp_path):
    tmp = str(tmp_path)
    if shutil.which("gcc") is None or not _gcc_sanitizers_work(tmp):
        pytest.skip("gcc with AddressSanitizer / UBSan runtimes not available")
    exe = os.path.join(tmp, "oracle_san")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_main.c"),
           "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


@pytest.mark.skipif(not _no_gpu_visible(), reason="expects the HIP runtime to find no device")
def test_c_abi_host_paths_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    tmp = str(tmp_path)
    csrc = os.path.join(ROOT, "q4_quantized_matvec_amd", "csrc")
    srcs = [os.path.join(ROOT, "tests", "abi_sanitize.cpp")] + sorted(
        os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    base = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *shlex.split(HOST_SAN),
            "-I", os.path.join(ROOT, "include"), "-I", csrc]

    def compile_one(src):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        r = subprocess.run(base + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(tmp, "abi_san")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *shlex.split(HOST_SAN), "-o", exe, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "ok" in r.stdout
