"""Build ``liblosa.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m block_sparse_attention_losa_amd.build`` (or call
:func:`build`).  Every call recompiles.

``python -m block_sparse_attention_losa_amd.build --lds-poison`` builds the
LDS-poison debug library, ``liblosa_poison.so`` beside ``liblosa.so``: the
same sources with ``LOSA_LDS_POISON`` defined, so that the attention kernels
fill their LDS with NaN bit patterns before each walk over the tiles and
before every tile slot is refilled (attn_common.h).  A GPU test runs the
path through both libraries and requires the same output bits.  It is a
checking build, never the product.

``python -m block_sparse_attention_losa_amd.build --host-sanitizers``
builds instead a CPU-side test library, ``_build/asan/liblosa_asan.so``:
the host code of every source with AddressSanitizer and
UndefinedBehaviorSanitizer (the device code is built as usual, without
them).  It is loaded through ``LOSA_LIBRARY`` with the sanitizer runtime
preloaded (:func:`sanitizer_runtime`), to run the C-ABI's host-side checks
under the sanitizers on a machine without a GPU; it is never used on one.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblosa.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIP_SOURCES = ["attn_bf16.hip", "attn_fwd.hip", "select.hip", "mass_fold.hip",
               "frozen_lists.hip", "noalloc.hip"]
HOST_SOURCES = ["losa_api.cpp"]

ARCH = "gfx950"
# packed fp32 VALU ops stay off: the compiler would otherwise pair float
# arithmetic into v_pk_* instructions
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}"] + DEVICE_FLAGS
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


POISON_DIR = os.path.join(OBJ_DIR, "poison")
POISON_LIB = os.path.join(PKG, "liblosa_poison.so")


def _compile_poison(src: str) -> str:
    obj = os.path.join(POISON_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-DLOSA_LDS_POISON"]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}"] + DEVICE_FLAGS
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_poison(verbose: bool = False) -> str:
    """The LDS-poison debug library (see the module doc)."""
    os.makedirs(POISON_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile_poison, HIP_SOURCES + HOST_SOURCES))
    tmp = POISON_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, POISON_LIB)
    if verbose:
        print(f"built {POISON_LIB}")
    return POISON_LIB


ASAN_DIR = os.path.join(OBJ_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "liblosa_asan.so")
# host code only; each sanitizer flag is scoped to the host compilation
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile_sanitized(src: str) -> str:
    obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + SANITIZE
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}"] + DEVICE_FLAGS
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """The CPU-side test library with host sanitizers (see the module doc)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile_sanitized, HIP_SOURCES + HOST_SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
           "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of the compiler was not found")
    return path


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, HIP_SOURCES + HOST_SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv[1:]:
        build_sanitized(verbose=True)
    elif "--lds-poison" in sys.argv[1:]:
        build_poison(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
