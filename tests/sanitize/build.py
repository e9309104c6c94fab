"""Host-side sanitizer builds used by tests/test_sanitizers.py (CPU only).

* the oracle's C loop nests (oracle/tp_mlp_oracle.c) with gcc and
  AddressSanitizer + UndefinedBehaviorSanitizer, linked into
  oracle_driver.c;
* the C ABI's argument-check layer (the library's api.hip), with both
  sanitizers on the host pass,
  linked into abi_driver.cpp, whose stub launchers abort if a call ever
  gets past the checks.

Every sanitizer flag applies to host code only.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "tensor_transformer_mlp_02_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["address", "undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")


def build_oracle_driver(out_dir: str) -> str:
    exe = os.path.join(out_dir, "oracle_driver")
    san = [f"-fsanitize={s}" for s in SAN]
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fno-sanitize-recover=all", *san, "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "tp_mlp_oracle.c"),
          "-lm"])
    return exe


def build_abi_driver(out_dir: str) -> str:
    exe = os.path.join(out_dir, "abi_driver")
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              "--offload-arch=gfx950", "-Xarch_host", "-fno-sanitize-recover=all", *host_san,
              "-I", CSRC]
    objs = []
    # api.hip keeps its device side (the allocation-free call's scratch
    # array lives there); the driver is host code only
    for src, extra in ((os.path.join(CSRC, "api.hip"), []),
                       (os.path.join(HERE, "abi_driver.cpp"), ["--cuda-host-only"])):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        _run([hipcc, *common, *extra, "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    _run([clang, *[f"-fsanitize={s}" for s in SAN], "-o", exe, *objs,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    return exe


if __name__ == "__main__":
    import tempfile
    d = tempfile.mkdtemp()
    print(build_oracle_driver(d))
    print(build_abi_driver(d))
