"""Build libtp_mlp.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m tensor_transformer_mlp_tp_amd.build`` or ``build()``.
Every call recompiles; objects go to ``_build/`` at the repository root.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libtp_mlp.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["abi.cpp", "reduce.hip", "decode.hip", "prefill.hip", "fp32.hip", "quant.hip", "gemv.hip"]

ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-I" + INCLUDE, "-I" + CSRC,
    # exact fp32 semantics: keep subnormals, no fast-math
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    # no packed-fp32 instructions in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain is required to build the library)")


def _compile(src, verbose, defines=(), build_dir=BUILD_DIR):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "--offload-arch=" + ARCH] + COMMON_FLAGS + ["-D" + d for d in defines] + \
        ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (src, r.stdout, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose=False, jobs=None, defines=(), out=LIB_PATH):
    """Compile every source and link libtp_mlp.so (next to this file by default).

    ``defines`` are extra preprocessor definitions (launch-shape variants);
    ``out`` is the library path to write.
    """
    build_dir = BUILD_DIR if not defines else os.path.join(BUILD_DIR, "v_" + "_".join(defines).replace("=", ""))
    os.makedirs(build_dir, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
