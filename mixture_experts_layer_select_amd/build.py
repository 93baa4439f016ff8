"""Build libmoe.so (the C-ABI MoE layer library) for gfx950 with hipcc.

Objects go to _build/ at the repository root; the shared library lands next
to this file so that it travels with the source tree.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["api.cpp", "partition.cpp", "route.hip", "permute.hip", "ffn.hip", "combine.hip", "rebalance.hip",
           "fused.hip"]


def _compile(src: str, verbose: bool, extra=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noisy = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noisy and verbose:
        print("\n".join(noisy))
    return obj


def build(verbose: bool = False, extra=(), out: str = OUT) -> str:
    """Compile every source and link the library; `extra` flags and `out`
    allow side builds (e.g. -D tuning variants) next to the default one."""
    build_dir = BUILD if out == OUT else os.path.join(BUILD, os.path.basename(out) + ".d")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
