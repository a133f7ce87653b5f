"""Build ``libtwotower.so`` in-tree with hipcc for gfx950.

Usage: ``python -m two_tower_cross_amd.build`` (or ``build()`` from Python). Always recompiles.
``--host-sanitized`` builds the host code under ASan/UBSan instead, ``--phase-stamps`` the
profiling build with per-work-group phase stamps.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtwotower.so")
ARCH = os.environ.get("TWOTOWER_ARCH", "gfx950")

# Packed fp32 VALU instructions are disabled for every device compile.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]

DEVICE_SOURCES = ["block_attn.hip", "unmask.hip", "linear.hip", "kv_append.hip", "probe.hip"]
# Per-source extra flags. The attention kernels run with the IEEE mode bit off: their max
# reductions then need no NaN-quieting instruction per operand (no input of theirs is a
# signaling NaN; NaN outputs for invalid sequences are written explicitly).
SOURCE_FLAGS = {"block_attn.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}
HOST_SOURCES = ["api.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        jobs.append([hipcc, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(OBJ, src + ".o")])
    for src in HOST_SOURCES:
        jobs.append([hipcc, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o",
                     os.path.join(OBJ, src + ".o")])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
          *[os.path.join(OBJ, s + ".o") for s in DEVICE_SOURCES + HOST_SOURCES]])
    os.replace(tmp, LIB)
    return LIB


STAMPS_LIB = os.path.join(OBJ, "libtwotower_stamps.so")


def build_phase_stamps() -> str:
    """The profiling build: the same sources compiled with TT_PHASE_STAMPS, so that the attention
    and projection kernels record per-work-group phase times (read by
    ``python -m two_tower_cross_amd.phases``). Never loaded by the tests, the smoke run or the
    bench. Returns its path."""
    hipcc = _hipcc()
    obj = os.path.join(OBJ, "stamps")
    os.makedirs(obj, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        jobs.append([hipcc, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-DTT_PHASE_STAMPS", "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(obj, src + ".o")])
    for src in HOST_SOURCES:
        jobs.append([hipcc, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o",
                     os.path.join(obj, src + ".o")])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(_run, jobs))
    tmp = STAMPS_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
          *[os.path.join(obj, s + ".o") for s in DEVICE_SOURCES + HOST_SOURCES]])
    os.replace(tmp, STAMPS_LIB)
    return STAMPS_LIB


SANITIZED_LIB = os.path.join(OBJ, "libtwotower_hostsan.so")


def build_host_sanitized() -> str:
    """The C ABI's host code (api.cpp: argument checks, planning, workspace sizing) built with g++
    under AddressSanitizer and UndefinedBehaviorSanitizer, the device launchers replaced by stubs
    that report no device (csrc/host_stubs.cpp). Load it with the sanitizer runtime preloaded
    (LD_PRELOAD of gcc's libasan) and TWOTOWER_LIB pointing to it. Returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = SANITIZED_LIB + ".tmp"
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=undefined", f"-I{rocm}/include", f"-I{CSRC}",
          os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_stubs.cpp"),
          f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib", "-o", tmp])
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    elif "--phase-stamps" in sys.argv:
        print(build_phase_stamps())
    else:
        print(build(verbose="-v" in sys.argv))
