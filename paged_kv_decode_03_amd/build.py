"""Build libpa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Each translation unit under csrc/ is compiled separately (in parallel), then
linked into paged_kv_decode_03_amd/libpa.so. Run ``python
paged_kv_decode_03_amd/build.py`` (as a file: importing the package loads the
library being built); ``__graft_entry__.build()`` loads this file by path.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"
SOURCES = ["pa_api.cpp", "pa_write.hip", "pa_decode_valu.hip", "pa_decode_mfma.hip",
           "pa_reduce.hip", "pa_copy.hip", "pa_prefill.hip"]
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # rounding exactly as written: fused multiply-adds only where fmaf() says so
    "-ffp-contract=off",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


# Per-source flags. pa_prefill.hip: MFMA accumulators in VGPRs (its output
# accumulators would otherwise live in AGPRs and be copied to VGPRs and back on
# every KV tile around the softmax rescale).
SOURCE_FLAGS = {"pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *CXXFLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "--hip-link" not in ln and ln.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")


def build(out: str = LIB, jobs: int = 8) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = out + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
