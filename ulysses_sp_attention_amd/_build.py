"""Build libulysses.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libulysses.so")
SOURCES = ["api.cpp", "exchange.hip", "attn_fwd.hip", "attn_f32.hip", "attn_bwd.hip", "attn_merge.hip",
           "logits_loss.hip", "tiled_mlp.hip", "noalloc.hip", "gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the generated code.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall",
]
# The kernels work on their matrix-core accumulators with vector
# instructions (softmax, masks, the loss epilogue) and run two or more waves
# per SIMD, so they keep them in ordinary VGPRs.
VGPR_FORM_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *VGPR_FORM_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def build_lib(jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libulysses.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_lib())
