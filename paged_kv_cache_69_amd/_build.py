"""Build libpa.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")
OBJ_DIR = os.path.join(PKG_DIR, "_build")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed-FP32 VALU forms stay disabled in every HIP build of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Extra flags per source. The prefill kernel rescales its MFMA accumulators with vector-ALU code
# inside its loop; with the accumulators in AGPRs the compiler would copy all of them to VGPRs and
# back on every tile, so that file uses the VGPR form of the MFMA instructions.
FILE_FLAGS = {
    "pa_prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libpa.so")
    return exe


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


_NOISE = "packed-fp32-ops' is not a recognized feature"


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if _NOISE not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    return log


def build(verbose: bool = False) -> str:
    """Compile every HIP source to an object (in parallel), link them into
    ``paged_kv_cache_69_amd/libpa.so``; return its path."""
    from concurrent.futures import ThreadPoolExecutor

    inc = ["-I", os.path.join(ROOT, "include")]
    # a fixed object directory: the paths hipcc records stay the same from build to build, so the
    # library is byte-reproducible (its hash identifies the code a profile was taken from)
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        flags = FILE_FLAGS.get(os.path.basename(src), [])
        jobs.append((obj, [hipcc(), *HIP_FLAGS, *flags, *inc, "-c", src, "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        logs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]))
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
