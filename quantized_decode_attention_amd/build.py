"""Builds libkvq.so for gfx950 with hipcc (in-tree, next to this file).

Flags: every HIP translation unit is compiled without packed-fp32 ops; the
quantizer's unit additionally with -ffp-contract=off so its fp32 steps stay
separate IEEE operations (bit-exact codes).  No fast-math anywhere.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = ["--offload-arch=gfx950"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(HERE, "..", "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
# (object name, source, extra flags)
UNITS = [
    ("kvq_quant", "kvq_quant.hip", ["-ffp-contract=off"]),
    # MFMA accumulators in VGPRs: keeps the O tiles out of AGPR<->VGPR copies
    # around the (rare) softmax rescale.
    ("kvq_decode", "kvq_decode.hip", MFMA_VGPR),
    ("kvq_bq2_quant", "kvq_bq2_quant.hip", ["-ffp-contract=off"]),
    ("kvq_bq2_decode", "kvq_bq2_decode.hip", MFMA_VGPR),
    ("kvq_api", "kvq_api.cpp", []),
    ("kvq_probe", "kvq_probe.hip", []),
    ("kvq_noalloc", "kvq_noalloc.hip", []),
]
# the decode partial kernels: one instantiation set per head dim, key bits and
# cache form, each its own object (they compile in parallel)
for _paged in (0, 1):
    for _d in (64, 128):
        for _bk in (2, 4, 8):
            _name = f"decode_partial_{'paged_' if _paged else ''}d{_d}_k{_bk}"
            UNITS.append((_name, "kvq_decode_inst.hip",
                          MFMA_VGPR + [f"-DKVQ_D={_d}", f"-DKVQ_BK={_bk}",
                                       f"-DKVQ_PAGED={_paged}", f"-DKVQ_INST={_name}"]))


def scratch_kernels(remarks: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) of every decode partial kernel (either format)
    that the compiler's resource-usage remarks report with scratch."""
    out, func = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            func = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0 and func and "partial" in func:
            out.append((func, int(m.group(1))))
    return out


def _compile(name: str, source: str, extra: list[str]) -> str:
    src = os.path.join(CSRC, source)
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if source.endswith(".hip") else []
    # the decode partial kernels (both formats) keep all their state in
    # registers: a kernel that needs scratch (a private array, an outlined
    # helper taking the wave state by reference, or spills under a waves-per-SIMD
    # target) runs many times slower, so it fails the build
    guard = name.startswith("decode_partial") or name == "kvq_bq2_decode"
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if guard else []
    cmd = [HIPCC, *ARCH, *COMMON, *extra, *remarks, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on " + name)
    if guard:
        bad = scratch_kernels(r.stderr)
        if bad:
            func, nbytes = bad[0]
            raise RuntimeError(f"{name}: {func} uses {nbytes} bytes/lane of scratch")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(UNITS), os.cpu_count() or 8, 16)) as ex:
        objs = list(ex.map(lambda u: _compile(*u), UNITS))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
