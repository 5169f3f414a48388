"""Build libstca.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m recsys_ultra_long_amd.build`` (or ``build()``).  Every
source in ``csrc/`` is compiled to an object in ``_build/`` in parallel, then
linked into ``recsys_ultra_long_amd/libstca.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libstca.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source flags.  attn.hip: no NaN reaches the attention (masked keys get
# a large finite negative score), so max() needs no NaN-quieting moves.
FILE_FLAGS = {"attn.hip": ["-fno-honor-nans"]}


def sources(src_dir: str = CSRC):
    return sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir)
                  if f.endswith((".hip", ".cpp")))


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libstca.so")
    return h


def _compile(src: str, extra, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True, extra=None, jobs: int = 8, out=None, src_dir=None) -> str:
    """Compile every source of ``src_dir`` (default csrc/) and link ``out``
    (default the in-tree libstca.so)."""
    src_dir = src_dir or CSRC
    lib_path = out or LIB
    obj_dir = OUT_DIR if src_dir == CSRC else os.path.join(OUT_DIR, "v_" + str(abs(hash(src_dir))))
    os.makedirs(obj_dir, exist_ok=True)
    extra = list(extra or [])
    srcs = sources(src_dir)
    with ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, obj_dir), srcs))
    tmp = lib_path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build()
