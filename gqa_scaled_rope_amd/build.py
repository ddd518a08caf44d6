"""Build libgqa_rope.so in-tree with hipcc for gfx950.

    python -m gqa_scaled_rope_amd.build        (or __graft_entry__.build())

Each .hip source is compiled to an object in parallel, then linked into
gqa_scaled_rope_amd/libgqa_rope.so next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa_rope.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the backend from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file code-generation options: no NaN is assumed in the prefill stream kernel, so row maxima
# need no quieting instruction (infinities are kept: masked scores are -inf).
FILE_FLAGS = {
    "attn_prefill_stream.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host sanitizers: the C-ABI layer (argument checks, the host-side rotary frequencies) rebuilt
# with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (each -fsanitize=
# goes to the host compilation; the device code is unchanged) and linked with the kernel objects
# of the normal build, for the CPU tests of the ABI (no kernel is launched there).
SANITIZED_SOURCES = ("gqa_api.hip", "rope_tables.hip")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of the AddressSanitizer runtime of hipcc's clang (to preload into a host process)."""
    base = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib", "llvm",
                        "lib", "clang")
    for root in (base, "/opt/rocm/llvm/lib/clang"):
        if os.path.isdir(root):
            for ver in sorted(os.listdir(root), reverse=True):
                p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(p):
                    return p
    return None


def build_sanitized(dest):
    """libgqa_rope with sanitized host code in directory dest (the normal build's objects are
    reused for the other sources); returns the library's path."""
    os.makedirs(dest, exist_ok=True)
    objs = []
    for src in sources():
        name = os.path.basename(src)
        if name in SANITIZED_SOURCES:
            obj = os.path.join(dest, name[:-4] + ".o")
            cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(name, []), *SANITIZE_FLAGS, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        else:
            obj = os.path.join(OBJ, name[:-4] + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} missing: run build() first")
        objs.append(obj)
    lib = os.path.join(dest, "libgqa_rope_sanitized.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
