"""Build liblca.so (gfx950) in-tree with hipcc.

    python long_context_attention_20_amd/build.py   (a plain script: importing the
    package itself needs the built library)

Every call recompiles: each source file is compiled to an object on its own
(in parallel), then the objects are linked into the shared library.  No
source refers to another's device code, so no device-side link is needed.
Packed-fp32 VALU ops are disabled for all device code.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "liblca.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = os.environ.get("LCA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblca)")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, err


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cc = hipcc()
    cmds = [[cc] + _flags() + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    for (rc, err), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([cc, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp] + objs, verbose)
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
