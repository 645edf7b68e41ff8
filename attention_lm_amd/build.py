"""Build libhymba_mixer.so (HIP, gfx950) in-tree with hipcc.

Each .hip source is compiled to an object in parallel, then linked into one
shared library next to this file. The output is replaced atomically.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhymba_mixer.so")
SOURCES = ["api.hip", "fuse.hip", "ssm.hip", "ssd.hip", "attn.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # never form packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax rescale and the epilogue
    # work on them with VALU instructions, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libhymba_mixer.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def sanitizer_runtime_dir() -> str:
    """Directory of the compiler's AddressSanitizer runtime (for LD_PRELOAD)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    base = os.path.join(llvm if os.path.isdir(llvm) else "/opt/rocm/llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True):
        d = os.path.join(base, ver, "lib", "linux")
        if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")):
            return d
    raise RuntimeError("AddressSanitizer runtime not found")


def build_host_sanitized(out_dir: str) -> str:
    """The same library with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged): for running the
    host-side argument checks under the sanitizers on a machine without a GPU.
    Load it with the ASan runtime preloaded. Returns the library path."""
    cc = hipcc()
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + san
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    lib = os.path.join(out_dir, "libhymba_mixer_hostsan.so")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, "-Xarch_host", "-shared-libsan", "-o", lib, *objs])
    return lib


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
