"""Build libdsa_indexer.so (HIP, gfx950) in-tree.

    python -m dsa_lightning_indexer_amd.build

compiles every source under csrc/ with hipcc for gfx950 and links
dsa_lightning_indexer_amd/lib/libdsa_indexer.so.  Objects go to _build/.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdsa_indexer.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "kernels_logits.hip", "kernels_topk.hip",
           "kernels_kwrite.hip", "kernels_handoff.hip", "kernels_chunk.hip",
           "kernels_calib.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed fp32 instructions disabled; IEEE fp32
# division and square root (the q quantisation relies on correctly rounded
# division to match its bit-exact definition).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-fno-gpu-rdc"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + ["-x", "hip", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    return obj, r.returncode, " ".join(cmd), msg


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, rc, cmd, msg in results:
        if verbose or rc:
            print(cmd)
            if msg:
                print(msg)
        if rc:
            raise RuntimeError(f"hipcc failed for {obj}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + \
        [o for o, _, _, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
