"""Build libbsa.so in-tree with hipcc for gfx950.

Usage: python -m video_dit_block_bsa_amd.build [--asm]
Every HIP source is compiled on each call (seconds per file); the shared
library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsa.so")
SOURCES = ["api.hip", "pool.hip", "select.hip", "attention.hip", "backward.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results go to arch VGPRs: every kernel feeds its accumulators to
    # VALU code (softmax, probabilities, epilogues) and fits in 256 VGPRs per
    # wave, so AGPR results would only add a copy per value.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, save_asm: str | None = None) -> str:
    """Compile every source (in parallel, one hipcc per file) and link
    libbsa.so; returns the library path."""
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="bsa_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if save_asm:
                os.makedirs(save_asm, exist_ok=True)
                cmd += ["-save-temps"]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True, cwd=save_asm or tmp)
            errs = "\n".join(
                l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l
            )
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
            if errs.strip() and verbose:
                print(errs, file=sys.stderr)
            return obj

        jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    asm_dir = None
    if "--asm" in sys.argv:
        asm_dir = os.path.join(ROOT, "_work", "asm")
    print(build(verbose=True, save_asm=asm_dir))
