"""Build ``liblowbit.so`` (the gfx950 HIP kernels and their C ABI) in-tree.

Every source is compiled with hipcc for gfx950 only.  Flags that matter for
the numerics: fp32 division and square root correctly rounded, denormals
kept, packed-fp32 instructions disabled (the compiler may not form
v_pk_*_f32 on its own).
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
SOURCES = ["abi.hip", "quantize.hip", "gemv.hip", "gemv2.hip", "gemv3.hip", "gemv4.hip", "gemv8.hip", "gemv_mma.hip", "gemm.hip", "gptq.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=on", "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def library_path() -> str:
    return os.path.join(HERE, "liblowbit.so")


def _obj_dir() -> str:
    d = os.path.join(ROOT, "_build")
    os.makedirs(d, exist_ok=True)
    return d


def _compile(src: str) -> str:
    obj = os.path.join(_obj_dir(), os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    out = library_path()
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
