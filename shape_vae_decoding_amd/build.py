"""Build libvdm.so (HIP for gfx950) in-tree: every csrc/*.hip compiled to an
object under _build/, then linked into shape_vae_decoding_amd/libvdm.so; then the
bounds-checked build (-DVDM_DEBUG=1) into shape_vae_decoding_amd/libvdm_debug.so.

    python shape_vae_decoding_amd/build.py

build_sanitized(out_dir) builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code (device code is compiled as usual)
into out_dir/libvdm_asan.so, for host-side checks of the C ABI.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvdm.so")
LIB_DEBUG = os.path.join(PKG, "libvdm_debug.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-FP32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# host code only (device code cannot take them): every sanitizer flag follows -Xarch_host
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _build_lib(lib: str, out_dir: str, extra=(), verbose: bool = True) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-o", tmp, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def build(verbose: bool = True) -> str:
    """The library, then its bounds-checked build (libvdm_debug.so: -DVDM_DEBUG=1)."""
    _build_lib(LIB, BUILD, verbose=verbose)
    _build_lib(LIB_DEBUG, os.path.join(BUILD, "debug"), ["-DVDM_DEBUG=1"], verbose=verbose)
    return LIB


def build_sanitized(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = ["-g", *SAN_HOST]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, extra), srcs))
    lib = os.path.join(out_dir, "libvdm_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", *SAN_HOST, "-o", lib, *objs], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build()
