"""Builds libmoe.so (HIP for gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed fp32 instructions are disabled in the
device code (`-packed-fp32-ops`); the routing and dispatch sources are also built without
floating-point contraction (their fp32 arithmetic is specified operation by operation).
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
# the debug build: MOE_DEBUG_CHECKS makes the kernels check the device-side preconditions
# (caller-supplied expert ids in [0, E) and distinct within a token) into a status word
# read by moe_debug_status
BUILD_DEBUG = os.path.join(HERE, "_build_debug")
LIB_DEBUG = os.path.join(HERE, "libmoe_debug.so")
SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "combine.hip", "pack.hip", "ffn_bf16.hip",
           "ffn_f32.hip", "quant_fp8.hip", "ffn_fp8.hip", "backward.hip"]
NO_CONTRACT = {"route.hip", "dispatch.hip"}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON]
    if debug:
        cmd.append("-DMOE_DEBUG_CHECKS")
    if src in NO_CONTRACT:
        cmd.append("-ffp-contract=off")
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Builds libmoe.so (or, with debug, libmoe_debug.so) and returns its path."""
    out_dir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
