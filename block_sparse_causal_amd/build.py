"""Build libtsa.so in-tree with hipcc for gfx950.

    python block_sparse_causal_amd/build.py

(run as a file: importing the package first would load the library being rebuilt)

Every source under csrc/ is compiled to an object in _build/ (in parallel) and
linked into block_sparse_causal_amd/libtsa.so.  Always rebuilds.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtsa.so")
ARCH = os.environ.get("TSA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["attention_fwd.hip", "attention_fwd_duo.hip", "attention_bwd.hip", "schedule_build.hip", "schedule_transpose.hip", "schedule_refine.hip", "tsa_api.cpp"]

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around VALU work)
    "-mllvm",
    "-amdgpu-mfma-vgpr-form=1",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtsa)")


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in proc.stdout.splitlines() if "is not a recognized feature for this target" not in line
    )
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


# Per-source extra flags.  The attention forward kernels take no NaN inputs by
# contract (their scores' max then needs no NaN quieting of the MFMA results).
EXTRA = {
    "attention_fwd.hip": ["-fno-honor-nans"],
    "attention_fwd_duo.hip": ["-fno-honor-nans"],
}


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
