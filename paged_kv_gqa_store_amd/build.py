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
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libpkv.so"
SOURCES = ["pkv_api.hip", "pkv_store.hip", "pkv_decode.hip", "pkv_decode_mfma.hip", "pkv_decode_rows.hip",
           "pkv_prefill.hip"]
# copy kernels that bound the store (bench.py's ceilings), a library of their own
BENCH_LIB = PKG / "libpkv_bench.so"
BENCH_SOURCES = ["pkv_bench.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]
# Per-source extras.  The prefill kernel keeps its matrix-core accumulators
# in ordinary VGPRs (the accumulator-register form costs a copy in and out of
# every rescaled accumulator each K/V tile).
SOURCE_FLAGS = {"pkv_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def _run(procs, verbose):
    errs = []
    for cmd, pr in procs:
        out, err = pr.communicate()
        err = "\n".join(line for line in err.splitlines() if NOISE not in line)
        if pr.returncode != 0:
            errs.append(f"hipcc failed ({pr.returncode}): {' '.join(cmd)}\n{err}")
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if errs:
        raise RuntimeError("\n".join(errs))


def build(verbose: bool = False) -> Path:
    """Compile every source to an object (in parallel), then link libpkv.so
    and libpkv_bench.so."""
    _build_lib(BENCH_LIB, BENCH_SOURCES, verbose)
    return _build_lib(LIB, SOURCES, verbose)


def _build_lib(lib: Path, sources, verbose: bool) -> Path:
    tmp = lib.with_suffix(f".so.tmp{os.getpid()}")
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as objdir:
        objs, procs = [], []
        for src in sources:
            obj = str(Path(objdir) / (Path(src).stem + ".o"))
            cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", str(CSRC / src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        _run(procs, verbose)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", str(tmp)]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run([(cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
