"""Builds libmuonh.so (the MuonH C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m orthogonalized_updates_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libmuonh.so"
SOURCES = ["muonh_abi.hip", "ns_gemm.hip", "elementwise.hip", "adamw.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmuonh.so)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # Keep the compiler from forming packed-fp32 VALU ops.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{ROOT / 'include'}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, jobs: int = 3, extra_flags=(), out: Path = LIB,
          objdir: Path = PKG / "_build") -> Path:
    """Compile every HIP source for gfx950 and link libmuonh.so (always rebuilds)."""
    cc = hipcc()
    objdir = Path(objdir)
    objdir.mkdir(parents=True, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = objdir / (Path(src).stem + ".o")
        objs.append(obj)
        cmd = [cc, *compile_flags(), *extra_flags, "-c", str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    out = Path(out)
    tmp = out.with_suffix(".so.tmp")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, out)
    return out


def _drain(procs: list) -> None:
    errors = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature: harmless.
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            errors.append(f"{src}:\n" + "\n".join(lines))
        elif lines:
            print(f"{src}:\n" + "\n".join(lines), file=sys.stderr)
    procs.clear()
    if errors:
        raise RuntimeError("HIP compilation failed:\n" + "\n\n".join(errors))


if __name__ == "__main__":
    print(build(verbose=True))
