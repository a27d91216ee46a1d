"""Build libsparse_attn.so and libsa_peaks.so (gfx950) in-tree with hipcc.

    python -m block_sparse_attention_08_amd.build      # or build() from Python

Compiles every ``csrc/*.hip`` to an object under ``_build/`` (in parallel) and
links them into ``block_sparse_attention_08_amd/lib/libsparse_attn.so``; the
measurement kernels under ``peaks/`` become ``lib/libsa_peaks.so``.  Both
libraries link against the HIP runtime that torch ships, so that a process
that imports torch first holds a single HIP runtime and torch's streams and
device pointers are valid inside them.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
BUILD = os.path.join(ROOT, "_build")
LIBNAME = "libsparse_attn.so"
PEAKS_DIR = os.path.join(PKG, "peaks")
PEAKS_LIBNAME = "libsa_peaks.so"
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 vector ALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file additions: the attention kernels produce and test no NaN (masked
# scores are -inf, inputs are finite), so their max reductions need no NaN
# quieting of cross-lane values.
FILE_FLAGS = {
    "attn_bf16.hip": ["-fno-honor-nans"],
    "attn_bf16_w16.hip": ["-fno-honor-nans"],
    "attn_bwd.hip": ["-fno-honor-nans"],
}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _torch_lib_dir() -> str | None:
    try:
        import torch  # noqa: F401
    except Exception:
        return None
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stdout + r.stderr


def _compile_and_link(srcs, tag, libname, verbose, jobs):
    hipcc = _hipcc()
    objs = [os.path.join(BUILD, tag + "_" + os.path.basename(s)[:-4] + ".o") for s in srcs]

    def one(pair):
        src, obj = pair
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        return _run([hipcc, *CXXFLAGS, *extra, "-c", src, "-o", obj])

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for out in ex.map(one, zip(srcs, objs)):
            if verbose and out.strip():
                print(out)

    tmp = os.path.join(LIBDIR, libname + ".tmp")
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    tl = _torch_lib_dir()
    if tl:
        # bind to torch's bundled HIP runtime (one runtime per process)
        link += [f"-L{tl}", f"-Wl,-rpath,{tl}", "-Wl,--disable-new-dtags"]
    _run(link)
    os.replace(tmp, os.path.join(LIBDIR, libname))
    return os.path.join(LIBDIR, libname)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile and link both libraries; returns the path of libsparse_attn.so."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    path = _compile_and_link(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), "sa", LIBNAME,
                             verbose, jobs)
    _compile_and_link(sorted(glob.glob(os.path.join(PEAKS_DIR, "*.hip"))), "peaks",
                      PEAKS_LIBNAME, verbose, jobs)
    return path


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
