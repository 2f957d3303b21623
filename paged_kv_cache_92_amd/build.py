"""Build libpkv.so in-tree with hipcc for gfx950 (one shared library, C ABI)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")

SOURCES = ["pkv_api.cpp", "cache_ops.hip", "decode.hip", "decode_gqa.hip", "prefill.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Per-source code-generation flags (none at present).
SOURCE_FLAGS: dict[str, list[str]] = {}

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 vector ops are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


OBJ_DIR = os.path.join(ROOT, "_build")


def build(verbose: bool = False, out: str = LIB, extra: tuple[str, ...] = ()) -> str:
    """Compile every source to an object (in parallel: each translation unit
    carries its own gfx950 code object), then link them into one library."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ_DIR, f"{tag}_{os.path.splitext(src)[0]}.o")
        cmd = [HIPCC, *compile_flags, *SOURCE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


# Host-side instrumentation: AddressSanitizer and UndefinedBehaviorSanitizer on
# the host pass only (each flag behind -Xarch_host), so device code is built
# exactly as in the regular library.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def host_asan_runtime() -> str:
    """The clang AddressSanitizer runtime a host-sanitized build needs preloaded."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError(f"no clang ASan runtime under {llvm}")
    return hits[-1]


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """libpkv whose host C++ (argument checks, schedule planning, workspace
    arithmetic, pkv_validate_host: pkv_api.cpp) runs under ASan + UBSan; the
    kernel objects are the regular build's (compiled first if absent).  Load
    it with host_asan_runtime() preloaded."""
    tag = os.path.splitext(os.path.basename(LIB))[0]
    objs = [os.path.join(OBJ_DIR, f"{tag}_{os.path.splitext(src)[0]}.o") for src in SOURCES
            if src != "pkv_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=verbose)
    api = out + ".api.o"
    compile_flags = [f for f in FLAGS if f not in ("-shared", "-O3")]
    cmd = [HIPCC, *compile_flags, "-O1", "-g", *HOST_SANITIZE, "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, "pkv_api.cpp"), "-o", api]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZE[:4],
           "-Xarch_host", "-shared-libasan", api, *objs, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


PROBE_SRC = os.path.join(PKG, "probe", "hbm_read_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libpkv_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The HBM read-ceiling probe bench.py runs (not part of libpkv.so)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
    sys.exit(0)
