"""Build libpkv.so (all HIP sources, gfx950 only) in-tree with hipcc.

    python -m paged_kv_gqa_store_amd.build

Packed-fp32 instructions are disabled in the device code
(``-target-feature -packed-fp32-ops``); the host pass warns that it does not
know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libpkv.so"
SOURCES = ["pkv_api.hip", "pkv_store.hip", "pkv_decode.hip", "pkv_decode_mfma.hip", "pkv_prefill.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
