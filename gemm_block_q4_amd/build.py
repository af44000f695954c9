"""Build step: compiles the HIP sources into ``libq4k.so`` for gfx950.

Run as ``python -m gemm_block_q4_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles: every source file is compiled
to an object in a temporary directory (in parallel), then the objects are
linked into the shared library.

``build(sanitize=True, out=...)`` makes the same library with AddressSanitizer
and UndefinedBehaviorSanitizer on the host code only (the argument checks,
workspace layout and launchers); device code is compiled as usual.  Such a
library must be loaded into a process that has the clang ASan runtime
preloaded (see :func:`asan_runtime`).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")

HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed FP32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SANITIZE_FLAGS = [
    "-g", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
]

# the host pass does not know the packed-fp32 feature and says so; that
# warning is harmless, anything else is shown
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def asan_runtime() -> str | None:
    """Path of the clang AddressSanitizer runtime that a sanitized build needs
    preloaded (None if the toolchain has none)."""
    pat = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang", "*", "lib",
                       "linux", "libclang_rt.asan-x86_64.so")
    found = sorted(glob.glob(pat)) or sorted(glob.glob(
        "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run(cmd: list[str]) -> list[str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    out = out or os.path.join(HERE, "libq4k_asan.so" if sanitize else "libq4k.so")
    flags = HIPCC_FLAGS + (SANITIZE_FLAGS if sanitize else [])
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="q4k_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in sources]
        cmds = [[cc, *flags, "-c", s, "-o", o] for s, o in zip(sources, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            msgs = [m for ms in pool.map(_run, cmds) for m in ms]
        tmp = out + ".tmp"
        link = [cc, *flags, "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        msgs += _run(link)
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
