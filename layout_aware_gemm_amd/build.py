"""Build the tgemm C-ABI shared library for gfx950 with hipcc (in-tree).

``python -m layout_aware_gemm_amd.build`` or ``build()`` compiles every
source under ``csrc/`` to an object in ``_build/`` (in parallel) and links
``layout_aware_gemm_amd/_lib/libtgemm.so``.  It always recompiles.
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
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libtgemm.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions in any kernel.
COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # only the extern "C" entry points are exported from the host side
    "-Xarch_host", "-fvisibility=hidden",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp")):
            out.append(os.path.join(CSRC, f))
    return out


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    msgs = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, msgs


def build(verbose=True, jobs=None):
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, msgs in ex.map(_compile, srcs):
            objs.append(obj)
            if verbose:
                for m in msgs:
                    print(m, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    # a library with unresolved symbols (e.g. a kernel whose host launch stub
    # was not emitted) must not replace a working one
    import ctypes

    ctypes.CDLL(os.path.abspath(tmp), mode=os.RTLD_NOW | os.RTLD_LOCAL)
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
