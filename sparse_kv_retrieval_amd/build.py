"""Build step: compile the HIP sources into sparse_kv_retrieval_amd/liblsa.so for gfx950.

Run as `python -m sparse_kv_retrieval_amd.build` or through `__graft_entry__.build()`.
It compiles every time it is called.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["score.hip", "score_stream.hip", "union.hip", "topk.hip", "gather.hip", "project.hip", "golden.hip", "train.hip", "lsa_api.hip"]
OUT = os.path.join(HERE, "liblsa.so")

BUILD_DIR = os.path.join(HERE, "_build")
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the epilogues read them without v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
SOURCE_FLAGS: dict = {}  # per-source additions to HIPCC_FLAGS
_NOISE = "is not a recognized feature for this target"


def _run(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for cmd, p in zip(cmds, procs):
        _, err = p.communicate()
        err = "\n".join(ln for ln in (err or "").splitlines() if _NOISE not in ln)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed ({p.returncode}): {' '.join(cmd)}\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    _run([[hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(s, []), *inc, "-c", os.path.join(HERE, "csrc", s), "-o", o]
          for s, o in zip(SOURCES, objs)], verbose)
    tmp = OUT + ".tmp"
    _run([[hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
