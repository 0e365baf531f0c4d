"""Build the HIP library ``_lib/libloop.so`` for gfx950 (hipcc, in-tree).

Every ``csrc/*.hip`` and ``csrc/*.cpp`` file is compiled to an object in
``_build/`` (in parallel), then linked into one shared library that links only
the HIP runtime.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "_lib", "libloop.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: no v_pk_*_f32 instructions are generated.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(HERE, "..", "include")]


def hip_runtime_dir() -> str:
    """Directory of the HIP runtime the process uses.  PyTorch-ROCm ships its
    own libamdhip64; the library links that one (by file name, with an rpath)
    so that a process holds exactly one HIP runtime."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is not None and spec.origin:
        d = os.path.join(os.path.dirname(spec.origin), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return "/opt/rocm/lib"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp"
    rt = hip_runtime_dir()
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang++"
    # -z defs: an unresolved symbol (e.g. a kernel whose host stub the
    # compiler did not emit) fails the link instead of the first dlopen
    subprocess.run([clang, "-shared", "-fPIC", "-o", tmp, *objs, "-L", rt, "-l:libamdhip64.so",
                    "-Wl,-rpath," + rt, "-Wl,-z,defs"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
