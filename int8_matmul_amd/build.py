"""Build libllm_int8.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python -m int8_matmul_amd.build [-v]

Each .hip source is compiled to an object in int8_matmul_amd/_build/ and
the objects are linked into int8_matmul_amd/libllm_int8.so, in tree, so the
library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libllm_int8.so")
SOURCES = ["quant.hip", "gemm.hip", "decode.hip", "decode_split.hip", "smoothquant.hip", "api.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # never let hipcc form packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and no FMA contraction in the scale arithmetic
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # a kernel whose host-side launch stub was not emitted leaves an
    # undefined symbol that only fails at load time: refuse it here
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    bad = [ln.split()[-1] for ln in und.stdout.splitlines() if "__device_stub__" in ln]
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the library: " + ", ".join(bad))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
