"""Build libdg.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdg.so")
ARCH = os.environ.get("DG_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops off: ordinary float code must not be turned into packed
# fp32 instructions (they are avoided on this hardware).
HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-file extra flags. Attention keeps its matrix-core accumulators in
# ordinary VGPRs: its softmax reads and rescales them on every key tile, and
# in the accumulator file every such access costs a register move.
EXTRA_FLAGS = {
    "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build_asan(verbose: bool = False) -> str:
    """A copy of the library whose host code (the C ABI: argument checks,
    workspace carving, launch sequences) is built with AddressSanitizer, in
    _build/libdg_asan.so for host-side tests; the device code is unchanged.
    Load it with the sanitizer runtime preloaded."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = []
    for src in srcs:
        if os.path.basename(src) == "api.hip":
            obj = os.path.join(BUILD, "api_asan.o")
            cmd = [hipcc(), *HIPFLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-c", src, "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("hipcc failed on api.hip (asan):\n" + res.stdout + res.stderr)
            objs.append(obj)
        else:
            objs.append(_compile(src, verbose))
    out = os.path.join(BUILD, "libdg_asan.so")
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-Xarch_host", "-fsanitize=address", *objs,
           "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed (asan):\n" + res.stdout + res.stderr)
    return out


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libdg.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
