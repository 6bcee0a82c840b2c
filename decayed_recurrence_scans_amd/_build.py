"""Build libdrs.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m decayed_recurrence_scans_amd._build`` or ``build()``.
The library lands in ``decayed_recurrence_scans_amd/_lib/libdrs.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_DIR = PKG / "_lib"
LIB = LIB_DIR / "libdrs.so"
OBJ_DIR = ROOT / "_build" / "drs"

SOURCES = ["api.hip", "wkv.hip", "ema.hip", "la_rec.hip", "combine.hip", "la_bwd.hip", "wkv_bwd.hip", "la_elem.hip", "la_rec_bwd.hip"] + [f"la_{t}_dk{d}.hip" for t in ("bf16", "f32") for d in (16, 32, 64, 128)] + [f"la_bidir_{t}_dk{d}.hip" for t in ("bf16", "f32") for d in (16, 32, 64)]
ARCH = os.environ.get("DRS_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def _compile(src: Path, obj: Path, verbose: bool):
    cmd = [hipcc(), *COMMON_FLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    """Compile every source and link libdrs.so; always recompiles."""
    OBJ_DIR.mkdir(parents=True, exist_ok=True)
    LIB_DIR.mkdir(parents=True, exist_ok=True)
    objs = [OBJ_DIR / (Path(s).stem + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, CSRC / s, o, verbose) for s, o in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
