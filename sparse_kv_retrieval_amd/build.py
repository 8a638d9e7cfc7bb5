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
SOURCES = ["score.hip", "score_stream.hip", "union.hip", "topk.hip", "gather.hip", "project.hip", "golden.hip",
           "train.hip", "lsa_api.hip"]
OUT = os.path.join(HERE, "liblsa.so")
# the streaming-read reference of the rooflines: a separate library, not part of lsa.h
PROBE_SOURCE = "probe.hip"
PROBE_OUT = os.path.join(HERE, "libprobe.so")

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
    ptmp = PROBE_OUT + ".tmp"
    _run([[hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
          [hipcc, *HIPCC_FLAGS, "-shared", os.path.join(HERE, "csrc", PROBE_SOURCE), "-o", ptmp]], verbose)
    os.replace(tmp, OUT)
    os.replace(ptmp, PROBE_OUT)
    return OUT


# Host-side sanitizers for the C-ABI validation layer: lsa_api.hip with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host code only (the GPU code is built as usual), linked with
# the kernel objects into a separate copy of the package. Only a CPU test loads it, with the
# sanitizer runtime preloaded; the product library is untouched.
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized_host(verbose: bool = False) -> str:
    """Build <SAN_DIR>/sparse_kv_retrieval_amd (liblsa.so with a sanitized host layer, and the binding)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "lsa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    pkg = os.path.join(SAN_DIR, "sparse_kv_retrieval_amd")
    os.makedirs(pkg, exist_ok=True)
    api = os.path.join(SAN_DIR, "lsa_api_san.o")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + SAN_FLAGS
    _run([[hipcc, *flags, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "csrc", "lsa_api.hip"),
           "-o", api]], verbose)
    _run([[hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, api, "-o", os.path.join(pkg, "liblsa.so")]],
         verbose)
    for f in ("__init__.py", "lsa.py"):
        with open(os.path.join(HERE, f), "rb") as src, open(os.path.join(pkg, f), "wb") as dst:
            dst.write(src.read())
    return pkg


# Debug build: the kernels that address rows through list entries check them against N_b
# (LSA_DEBUG_CHECKS=1; see lsa_debug_range_errors), in a separate copy of the package so that
# the product library is untouched. GPU tests load it in a child process.
DEBUG_DIR = os.path.join(HERE, "_debug")
DEBUG_SOURCES = ["score.hip", "gather.hip", "lsa_api.hip"]


def build_debug(verbose: bool = False) -> str:
    """Build <DEBUG_DIR>/sparse_kv_retrieval_amd (liblsa.so with the device range checks, and the binding)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s not in DEBUG_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    pkg = os.path.join(DEBUG_DIR, "sparse_kv_retrieval_amd")
    os.makedirs(pkg, exist_ok=True)
    dobjs = [os.path.join(DEBUG_DIR, s.replace(".hip", "_debug.o")) for s in DEBUG_SOURCES]
    _run([[hipcc, *HIPCC_FLAGS, "-DLSA_DEBUG_CHECKS=1", "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(HERE, "csrc", s), "-o", o] for s, o in zip(DEBUG_SOURCES, dobjs)], verbose)
    tmp = os.path.join(pkg, "liblsa.so.tmp")
    _run([[hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *dobjs, "-o", tmp]], verbose)
    os.replace(tmp, os.path.join(pkg, "liblsa.so"))
    for f in ("__init__.py", "lsa.py"):
        with open(os.path.join(HERE, f), "rb") as src, open(os.path.join(pkg, f), "wb") as dst:
            dst.write(src.read())
    return pkg


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_debug(verbose=True))
    if "--sanitized-host" in sys.argv:
        print(build_sanitized_host(verbose=True))
