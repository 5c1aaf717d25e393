"""Build libuno.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m lossless_diffusion_drafted_amd.build [--verbose]
"""

import concurrent.futures
import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libuno.so")

SOURCES = ["api.cpp", "verify.hip", "tv.hip", "gemm.hip", "model.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions are turned off for all device code: hipcc would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + lang + COMMON + DEVICE_FLAGS + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, cmd, r


def build(verbose=False):
    """Compile every source and link libuno.so; raises RuntimeError on failure."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src, obj, cmd, r in ex.map(_compile, srcs):
            if verbose or r.returncode != 0:
                sys.stderr.write(" ".join(cmd) + "\n")
                sys.stderr.write(_filter_noise(r.stdout + r.stderr))
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libuno.so failed")
    # a shared library links with unresolved symbols; loading it finds them now
    # rather than in the first call
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"libuno.so does not load: {e}")
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"built {LIB}\n")
    return LIB


def _filter_noise(text):
    # The host compilation pass does not know the device-only feature flag.
    return "".join(l for l in text.splitlines(True)
                   if "packed-fp32-ops' is not a recognized feature" not in l)


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
