"""Compile the HIP sources into the in-tree shared library ``libcpa.so`` (gfx950)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libcpa.so")
DIAG_LIB_PATH = os.path.join(PKG, "libcpa_diag.so")
DIAG_SOURCES = ("diag_mfma.hip",)   # measurement helpers (include/cpa_diag.h), a library of their own
SOURCES = ("block_union.hip", "block_plans.hip", "prefill_regstaged.hip", "prefill_bf16.hip", "prefill_direct.hip",
           "kv_append.hip", "cpa_api.hip")
ARCH = os.environ.get("CPA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# per-source extra flags
EXTRA = {"prefill_bf16.hip": ["-fno-honor-nans"], "prefill_direct.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libcpa.so (and the measurement helpers' libcpa_diag.so);
    always recompiles.  Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES + DIAG_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out, file=sys.stderr)
    for path, o in ((LIB_PATH, objs[:len(SOURCES)]), (DIAG_LIB_PATH, objs[len(SOURCES):])):
        tmp = path + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *o])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
