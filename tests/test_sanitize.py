"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host code: kvq_api.cpp (argument checks, sizes, error text,
  the HIP-failure path) built with the sanitizers on the host side only and
  linked with stand-in launchers that report no device (tests/sanitize), then
  driven by tests/sanitize/host_driver.cpp: a sweep of valid and invalid
  geometries through every size and check, null and out-of-range arguments,
  KVQ_ERR_HIP with the runtime's text, and per-thread error text read back
  by eight threads at once.
* The oracle: its C library rebuilt with the sanitizers
  (oracle.build_sanitized) and its pinned tests run against that build (the
  exhaustive fp32 -> fp16 sweep left out for time).
Any sanitizer report aborts the program, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm compilers")
def test_host_api_under_sanitizers(tmp_path):
    inc = os.path.join(ROOT, "include")
    # sanitizers on the host side only of the HIP translation units
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(ROOT, "quantized_decode_attention_amd", "csrc", "kvq_api.cpp"),
                os.path.join(HERE, "host_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", *host_san,
              "-I" + inc, "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "host_driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([CLANG, "-std=c++17", "-O1", "-g", *san, "-I" + inc, "-c",
          os.path.join(HERE, "host_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "host_driver")
    _run([CLANG, *san, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-lpthread", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=600)
    assert "host api under sanitizers: ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ, KVQ_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_attention.py", "test_oracle_bq2.py", "test_oracle_quantizer.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not exhaustive", *tests],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
