"""Build the gfx950 HIP library in-tree with hipcc (no JIT cache, no torch extension)."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
SOURCES = [PKG_DIR / "csrc" / n for n in ("verify_attn.hip", "compact.hip", "tree.hip")]
INCLUDE_DIR = REPO_DIR / "include"
LIB_PATH = PKG_DIR / "libverify_attn.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs: the partial kernel keeps Q (144 registers)
    # as an MFMA operand in AGPRs and its output accumulators in VGPRs; the
    # AGPR-result form makes the allocator copy the accumulators every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the leading scalar kernel arguments (up to 16 dwords) arrive preloaded
    # in scalar registers: the partial and merge kernels pass the pointers
    # their first loads need there, which saves one dependent load at entry
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(root) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build_library(force: bool = True, verbose: bool = False) -> Path:
    """Compile every HIP source into libverify_attn.so next to this file."""
    if not force and LIB_PATH.exists():
        return LIB_PATH
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE_DIR}", *map(str, SOURCES), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
