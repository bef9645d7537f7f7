"""Build librepro.so for gfx950 with hipcc (in-tree, no JIT).

Flags that are part of the numeric contract:
  -ffp-contract=off                 multiply and add are never fused (OPEN-1B,
                                    section 2.1 "Fused multiply-add")
  -packed-fp32-ops (disabled)       no v_pk_{add,mul,fma}_f32
  -fgpu-flush-denormals-to-zero     the VALU flushes subnormal operands and
                                    results (section 2.1 "Subnormals"); on
                                    gfx950 this is the x86 FTZ/DAZ rule.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librepro.so")
# Measurement support, not part of librepro: the VALU issue-rate streams that
# bench.py --valu-rates runs.
RATES_SRC = "valu_rates.hip"
RATES_LIB = os.path.join(PKG, "libvalu_rates.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
          "-fgpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{HERE}",
          "-Wno-unused-command-line-argument"]
SOURCES = {
    "api.cpp": ["-x", "hip"],
    "elementwise.hip": [],
    # Keep MFMA results in architectural VGPRs, where v_add_f32 reads them
    # directly (otherwise each product is first copied out of an AGPR).
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "state_hash.hip": [],
    "replay.hip": [],
    "fused.hip": [],
    "optimizer.hip": [],
}


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(HERE, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature and says so.
    err = "\n".join(ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = list(SOURCES.items()) + [(RATES_SRC, [])]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), jobs))
    rates_obj = objs.pop()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", rates_obj, "-o", RATES_LIB + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(RATES_LIB + ".tmp", RATES_LIB)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def disassemble(src: str = "gemm.hip") -> str:
    """AMD assembly of one of our own kernels (for the instruction-mix audit)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *COMMON, *SOURCES.get(src, []), "--cuda-device-only", "-S",
           os.path.join(HERE, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as fh:
        return fh.read()


if __name__ == "__main__":
    print(build(verbose=True))
