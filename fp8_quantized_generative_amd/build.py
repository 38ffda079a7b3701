"""Build the gfx950 HIP library ``librq_fp8.so`` in-tree with hipcc.

Each ``csrc/*.hip`` file is compiled to an object (in parallel) and the objects are linked
into one shared library next to this file.  Flags:

* ``--offload-arch=gfx950``: MI355X (CDNA4) only;
* ``-ffp-contract=off``: no implicit FMA contraction, so every rounding in the quantizer,
  the epilogue and the combine is the one written in the source;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed FP32 instructions.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "librq_fp8.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["quant.hip", "gemm.hip", "moe.hip", "router.hip", "attention.hip", "topk.hip", "layout.hip", "api.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (proc.returncode, " ".join(cmd), out))
    return out


def build(verbose=False, extra_flags=()):
    """Compile every HIP source and link ``librq_fp8.so``.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
