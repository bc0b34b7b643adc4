"""Build the HIP library (gfx950) and the host-only planning library, in-tree.

    python -m communication_gemm_role_amd.build [--sanitize-host]

libmk.so        every HIP translation unit of csrc/ plus the C ABI, for --offload-arch=gfx950
libmk_host.so   csrc/mk_host_check.cpp built with g++ alone (no HIP), for CPU tests of the
                argument validation and planning; --sanitize-host adds ASan/UBSan to it
_build/mk_host_plan_test   (tests only) csrc/mk_host_plan_test.cpp under ASan/UBSan, see
                build_host_plan_test
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmk.so")
HOSTLIB = os.path.join(PKG, "libmk_host.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 VALU ops
    # Clang copies a by-value kernel parameter struct into private memory and relies on InstCombine
    # to read it from the kernel-argument segment instead; InstCombine gives up past 300 uses of the
    # copy, which leaves the whole struct in scratch and every parameter read in the hot loops a
    # scratch load.  The role kernels use their parameters more often than that.
    "-mllvm", "-instcombine-max-copied-from-constant-users=4096",
    "-Rpass-analysis=kernel-resource-usage",  # per-kernel resource remarks, checked below
    "-I", INCLUDE, "-I", CSRC,
]
# A kernel's register spills or a scratch area the size of a parameter struct mean the hot loop
# reads memory it should not; the build refuses them.
MAX_SCRATCH_BYTES = 128
SOURCES = ["mk_ag_gemm.hip", "mk_gemm_reduce.hip", "mk_moe.hip", "mk_mlp.hip", "mk_ring_attn.hip", "mk_selftest.hip",
           "mk_api.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def check_resources(src: str, remarks: str) -> list:
    """Parse the kernel-resource-usage remarks of one compile; raise on spills or large scratch."""
    kernels, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|VGPRs Spill|"
                      r"LDS Size \[bytes/block\]): (\S+)", line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"kernel": val}
            kernels.append(cur)
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    for k in kernels:
        if k.get("VGPRs Spill", 0) > 0 or k.get("ScratchSize", 0) >= MAX_SCRATCH_BYTES:
            raise RuntimeError(f"{src}: kernel {k['kernel']} spills or uses scratch: {k}")
    return kernels


# Per-source extra flags.  Ring attention: keep MFMA operands and results in VGPRs (the kernel
# fits in 205 of them at one wave per SIMD); left to itself the compiler puts the score and output
# accumulators in AGPRs and copies them to VGPRs and back for every softmax step (~180 extra
# instructions per 64-key block).
SOURCE_FLAGS = {"mk_ring_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    out = _run([HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    check_resources(src, out)
    return obj


def build_gpu_lib(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_host_lib(sanitize: bool = False) -> str:
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-shared", "-fPIC", "-Wall", "-I", CSRC]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    tmp = HOSTLIB + ".tmp"
    _run(cmd + [os.path.join(CSRC, "mk_host_check.cpp"), "-o", tmp])
    os.replace(tmp, HOSTLIB)
    return HOSTLIB


PLAN_TEST = os.path.join(BUILD, "mk_host_plan_test")


def build_host_plan_test() -> str:
    """The CPU driver over the host planning functions (csrc/mk_host_plan_test.cpp), built with g++
    alone under AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal."""
    os.makedirs(BUILD, exist_ok=True)
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-Wall", "-I", CSRC, "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    tmp = PLAN_TEST + ".tmp"
    _run(cmd + [os.path.join(CSRC, "mk_host_plan_test.cpp"), "-o", tmp])
    os.replace(tmp, PLAN_TEST)
    return PLAN_TEST


def build(sanitize_host: bool = False) -> None:
    build_gpu_lib()
    build_host_lib(sanitize_host)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--sanitize-host", action="store_true")
    a = ap.parse_args()
    build(a.sanitize_host)
    print(LIB)
    print(HOSTLIB)
    sys.exit(0)
