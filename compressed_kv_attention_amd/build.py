"""Build libswa.so for gfx950 in-tree.

Each source under csrc/ is compiled with hipcc for gfx950 (packed fp32 vector
ops disabled), and the objects are linked into compressed_kv_attention_amd/
libswa.so against the HIP runtime that torch ships, so that the library and
torch share one runtime (and torch's stream handles) in the same process.

Usage:  python -m compressed_kv_attention_amd.build  [-v]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libswa.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["swa_api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "debug_visibility.hip", "pool_rope.hip", "chunk.hip", "backward.hip", "nsa.hip",
           "decode.hip"]
ARCH = os.environ.get("SWA_OFFLOAD_ARCH", "gfx950")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is required to link against its HIP runtime")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is expected
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libswa.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tlib = _torch_lib_dir()
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["g++", "-shared", "-o", tmp] + objs + [f"-L{tlib}", "-l:libamdhip64.so", f"-Wl,-rpath,{tlib}",
                                                  "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
