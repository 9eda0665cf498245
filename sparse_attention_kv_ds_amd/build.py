"""Build libds_indexer.so (gfx950) in-tree with hipcc.

Each source is compiled to an object in parallel, then linked into the shared
library next to this file.  Packed-fp32 VALU instructions are disabled for
every HIP source (they are not used by hand and must not be generated).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libds_indexer.so")
# the same sources with DSI_STAMPS: kernels also record phase timestamps
# (ds_indexer_stamps_read); for the phase breakdowns only, never the product
LIB_STAMPS = os.path.join(HERE, "libds_indexer_stamps.so")
SOURCES = ["api.cpp", "scorer.hip", "topk.hip", "attention.hip", "qproj.hip", "static_scratch.hip"]
# Extra flags per source.  The scorer is built without NaN semantics: its
# inputs are finite by contract, and with NaNs honoured every ReLU (fmaxf)
# costs an extra canonicalising instruction.
# MFMA accumulators are kept in ordinary VGPRs (the epilogue reads them with
# VALU instructions; in AGPRs every read would cost an extra move).
EXTRA = {"scorer.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attention.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "qproj.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")


def build_library(out: str = LIB, stamps: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libds_indexer.so (with
    stamps: the timestamped build, libds_indexer_stamps.so)."""
    if stamps and out == LIB:
        out = LIB_STAMPS
    defines = ("DSI_STAMPS",) if stamps else ()
    with tempfile.TemporaryDirectory(prefix="dsi_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            list(ex.map(lambda src, obj: _compile(src, obj, defines), SOURCES, objs))
        tmp_out = os.path.join(tmp, "libds_indexer.so")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        shutil.copyfile(tmp_out, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library())
    print(build_library(stamps=True))
