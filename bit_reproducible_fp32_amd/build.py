"""Builds librepops.so (gfx950) in-tree with hipcc, plus the device assembly
that the instruction scan in the tests reads.

Flags that matter for the arithmetic:

* ``-ffp-contract=off``: no multiply-add contraction anywhere (the kernels
  also carry ``#pragma clang fp contract(off)``);
* ``-fno-fast-math`` and ``-fno-gpu-flush-denormals-to-zero``: IEEE binary32
  with gradual underflow (kernel descriptors must say denorm mode 3);
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: binary32 ``/`` and ``sqrt``
  are the correctly rounded IEEE operations;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: the compiler must not
  form packed two-lane FP32 instructions.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librepops.so")
ASM = os.path.join(HERE, "librepops_gfx950.s")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

KERNEL_SOURCES = [os.path.join(CSRC, "repops_kernels.hip"), os.path.join(CSRC, "repops_fold.hip"),
                  os.path.join(CSRC, "repops_merkle.hip"), os.path.join(CSRC, "repops_ops.hip")]
SOURCES = KERNEL_SOURCES + [os.path.join(CSRC, "repops_api.cpp"),
                            os.path.join(CSRC, "repops_fold_api.cpp"),
                            os.path.join(CSRC, "repops_merkle_api.cpp"),
                            os.path.join(CSRC, "repops_ops_api.cpp")]

FP_FLAGS = ["-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
            "-fhip-fp32-correctly-rounded-divide-sqrt"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # matrix-instruction results land in ordinary VGPRs, where the
                # VALU adds read them (no accumulation-register copies)
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-command-line-argument"]


def _manifest_defines():
    flags = " ".join(FP_FLAGS + ["-packed-fp32-ops", "-O3"])
    return ["-DREPOPS_BUILD_FLAGS=\"%s\"" % flags, "-DREPOPS_OFFLOAD_ARCH=\"%s\"" % ARCH]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile every source into librepops.so and write the gfx950 assembly.

    The sources compile to objects in parallel, next to the device-only
    assembly of each kernel source (for the instruction scan); the objects
    then link into the library."""
    tag = "%d" % os.getpid()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + "." + tag + ".o")
        objs.append(obj)
        jobs.append([HIPCC, *COMMON, *FP_FLAGS, *DEVICE_FLAGS, *_manifest_defines(), "-c",
                     "-o", obj, src])
    asms = []
    for src in KERNEL_SOURCES:
        asm = os.path.join(objdir, os.path.basename(src) + "." + tag + ".s")
        asms.append(asm)
        jobs.append([HIPCC, *COMMON, *FP_FLAGS, *DEVICE_FLAGS, "--cuda-device-only", "-S",
                     "-o", asm, src])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
                f.result()
        tmp = LIB + ".tmp" + tag
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB)
        with open(ASM + ".tmp", "w") as f:
            f.write("\n".join(open(a).read() for a in asms))
        os.replace(ASM + ".tmp", ASM)
    finally:
        for path in objs + asms:
            if os.path.exists(path):
                os.remove(path)
        try:
            os.rmdir(objdir)
        except OSError:
            pass
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
