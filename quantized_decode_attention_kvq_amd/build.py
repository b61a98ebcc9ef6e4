"""Build libkvq.so (HIP kernels for gfx950 + the C-ABI host code) in-tree with hipcc.

Run as ``python quantized_decode_attention_kvq_amd/build.py`` (by path: importing the package
loads the library, which may be missing or stale before a build).  The quantize/calibration unit is
compiled with -ffp-contract=off so its binary32 operations round in the order written; every HIP
unit is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
BENCH_LIB = os.path.join(HERE, "libkvq_bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

ROOT = os.path.dirname(HERE)
INCLUDE = os.environ.get("KVQ_INCLUDE", os.path.join(ROOT, "include"))
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]
UNITS = [
    ("kvq_quant.hip", DEVICE + ["-ffp-contract=off"]),
    ("kvq_decode.hip", DEVICE),
    ("kvq_decode_mfma.hip", DEVICE + ["-ffp-contract=off"]),  # holds the fused append
    # matrix-core accumulators in VGPRs: the softmax rescales them with vector ALU instructions,
    # and AGPR-homed accumulators cost a copy each way per chunk
    ("kvq_prefill_attn.hip", DEVICE + ["-mllvm", "--amdgpu-mfma-vgpr-form"]),
    ("kvq_host.cpp", ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),  # host only
]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        objs = list(ex.map(lambda u: _compile(*u), UNITS))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # the measurement loop driver (calls the C ABI of libkvq.so; not part of that ABI)
    bobj = os.path.join(BUILD, "kvq_bench.o")
    for cmd in ([HIPCC, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, "kvq_bench.cpp"), "-o", bobj],
                [HIPCC, "-shared", "-fPIC", "-o", BENCH_LIB + ".tmp", bobj, f"-L{HERE}", "-lkvq",
                 "-Wl,-rpath,$ORIGIN"]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"bench driver build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
