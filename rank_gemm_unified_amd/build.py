"""Build liblorapool.so for gfx950 with hipcc, in-tree.

    python rank_gemm_unified_amd/build.py          (or __graft_entry__.build())

Run it by path: importing the package loads the library this script builds.

Every .hip file under csrc/ is compiled to an object under _build/ and linked into
rank_gemm_unified_amd/liblorapool.so.  Always recompiles.  A hash of the sources (csrc/ and
include/lorapool.h) is compiled in; lora_version() reports it and importing the package refuses a
library whose hash differs from the sources beside it.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
from _srchash import source_hash  # noqa: E402
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblorapool.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def _compile(src: str, src_hash: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, f'-DLORAPOOL_SRC_HASH="{src_hash}"', "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "(ignoring feature)" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    src_hash = source_hash()
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, src_hash), srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources (source hash {src_hash})")
    return LIB


if __name__ == "__main__":
    build()
