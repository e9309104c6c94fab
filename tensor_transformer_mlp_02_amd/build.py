"""Build libtpmlp.so (HIP kernels + C ABI) for gfx950 with hipcc.

Every HIP source is compiled with packed-fp32 instruction forms disabled
(the compiler otherwise forms v_pk_* fp32 arithmetic from ordinary float
code); the library is written for gfx950 only.

`--define NAME=VALUE` builds a variant with a build option set (e.g.
TP_TILE_ORDER, the GEMM tile placement) into a folder of its own,
_build_<hash of the options>/libtpmlp.so (or --out); the binding loads such
a library when TPMLP_LIBRARY names it.
"""
import argparse
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtpmlp.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.hip", "gemm_bf16.hip", "gemm_f32.hip", "partial_sum.hip", "moe.hip", "fp8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str, verbose: bool, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: that note is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), out=None) -> str:
    defines = list(defines)
    build_dir = BUILD_DIR
    if defines:
        tag = hashlib.sha256(" ".join(defines).encode()).hexdigest()[:12]
        build_dir = f"{BUILD_DIR}_{tag}"
    if out is None:
        out = os.path.join(build_dir, "libtpmlp.so") if defines else OUT
    if defines and os.path.abspath(out) == OUT:
        raise ValueError("a build with defines may not replace the default library")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    print(build(verbose=True, defines=a.define,
                out=None if a.out is None else os.path.abspath(a.out)))
