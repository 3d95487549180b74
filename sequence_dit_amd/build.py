"""Build the HIP library ``libas_attn.so`` in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled with hipcc to an object under ``_build/``
(in parallel), then linked into ``sequence_dit_amd/libas_attn.so``. hipcc
cross-compiles for gfx950 without a GPU. Usage: ``python -m sequence_dit_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libas_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Diagnostics library: the same, with the single-partition bf16 kernels built with
# -DAS_WG_STAMPS (per-workgroup timestamps; see sequence_dit_amd/wg_stamps.py).
STAMPS_LIB_PATH = os.path.join(PKG, "libas_attn_stamps.so")
STAMPS_SOURCE = "partition_attn.hip"
ARCH = "gfx950"

SOURCES = ["api.hip", "partition_attn.hip", "partition_attn_fp8.hip", "partition_attn_fp8v.hip", "partition_attn_grouped.hip", "merge.hip",
           "contribution.hip", "planner.hip"]

# Per-source flags. The attention kernels never see NaN (finite inputs, -inf only
# as a max/exp operand), so NaN-honouring max and IEEE-mode operand
# canonicalisation are switched off there: fmaxf becomes a single v_max/v_max3.
_ATTN_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
SOURCE_FLAGS = {"partition_attn.hip": _ATTN_FLAGS, "partition_attn_fp8.hip": _ATTN_FLAGS, "partition_attn_fp8v.hip": _ATTN_FLAGS,
                "partition_attn_grouped.hip": _ATTN_FLAGS}

# Packed fp32 VALU instructions are kept out of the device code on purpose: hipcc
# only emits them from ordinary float code, and the kernels do not need them.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    stamps_obj = os.path.join(BUILD_DIR, STAMPS_SOURCE.replace(".hip", "_stamps.o"))
    cmds.append([cc, *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(STAMPS_SOURCE, []), "-DAS_WG_STAMPS", "-c",
                 os.path.join(CSRC, STAMPS_SOURCE), "-o", stamps_obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    for path, objects in ((LIB_PATH, objs),
                          (STAMPS_LIB_PATH, [stamps_obj if os.path.basename(o) == STAMPS_SOURCE.replace(".hip", ".o")
                                             else o for o in objs])):
        tmp = path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objects], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
