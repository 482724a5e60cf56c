"""Compile the HIP sources of liblca.so for gfx950 (in-tree)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblca.so")
SOURCES = ["api.hip", "compress.hip", "indexer.hip", "attend.hip", "noalloc.hip"]
# the benchmark's ceiling measurements, a library of their own
PEAK_LIB = os.path.join(HERE, "libpeak.so")
PEAK_SOURCES = ["peak.hip"]
# keep MFMA accumulators in arch VGPRs where the kernel rescales them with VALU
EXTRA = {"attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 arithmetic anywhere (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, obj_dir), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAK_SOURCES], PEAK_LIB)
    if verbose:
        print("built", LIB, "and", PEAK_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
