"""Build libpa.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libpa_probe.so")  # the benchmark's measurement probes
TIMELINE_LIB_PATH = os.path.join(PKG_DIR, "libpa_timeline.so")  # per-wave timelines (built on request)
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
    # the matrix-rate probe measures what the prefill kernel's form of the instruction sustains; in the
    # AGPR form its fenced loop would also copy every accumulator after each MFMA
    "pa_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libpa.so")
    return exe


def sources(folder: str = "csrc") -> list[str]:
    return sorted(glob.glob(os.path.join(PKG_DIR, folder, "*.hip")))


_NOISE = "packed-fp32-ops' is not a recognized feature"


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if _NOISE not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{log}")
    return log


def _build_lib(folder: str, lib_path: str, logs: list, ex, defines=(), tag: str = "") -> None:
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in sources(folder):
        obj = os.path.join(OBJ_DIR, tag + folder + "_" + os.path.basename(src) + ".o")
        flags = FILE_FLAGS.get(os.path.basename(src), [])
        jobs.append((obj, [hipcc(), *HIP_FLAGS, *flags, *defines, *inc, "-c", src, "-o", obj]))
    logs += list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = lib_path + ".tmp"
    logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]))
    os.replace(tmp, lib_path)


def build(verbose: bool = False, timeline: bool = True) -> str:
    """Compile every HIP source to an object (in parallel) and link them: csrc/ into
    ``paged_kv_cache_69_amd/libpa.so`` (the decode library) and probe/ into ``libpa_probe.so`` (the
    benchmark's measurement probes) and, with ``timeline``, csrc/ again with PA_TIMELINE=1 into
    ``libpa_timeline.so`` (the per-wave timeline build); return the decode library's path."""
    from concurrent.futures import ThreadPoolExecutor

    # a fixed object directory: the paths hipcc records stay the same from build to build, so the
    # library is byte-reproducible (its hash identifies the code a profile was taken from)
    os.makedirs(OBJ_DIR, exist_ok=True)
    logs: list = []
    with ThreadPoolExecutor(max_workers=8) as ex:
        _build_lib("csrc", LIB_PATH, logs, ex)
        _build_lib("probe", PROBE_LIB_PATH, logs, ex)
        if timeline:
            _build_lib("csrc", TIMELINE_LIB_PATH, logs, ex, defines=("-DPA_TIMELINE=1",), tag="timeline_")
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB_PATH


def build_timeline(verbose: bool = False) -> str:
    """The measurement build: csrc/ with PA_TIMELINE=1 into ``libpa_timeline.so`` (the decode kernels
    also record a per-wave timeline; include/pa_timeline.h) alone."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    logs: list = []
    with ThreadPoolExecutor(max_workers=8) as ex:
        _build_lib("csrc", TIMELINE_LIB_PATH, logs, ex, defines=("-DPA_TIMELINE=1",), tag="timeline_")
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return TIMELINE_LIB_PATH


if __name__ == "__main__":
    import sys

    print(build_timeline(verbose=True) if "--timeline" in sys.argv[1:] else build(verbose=True))
