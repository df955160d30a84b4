"""Build ``libbitlinear.so`` (the C-ABI HIP library) and ``libblmeasure.so`` (the
benchmark's reference kernels) for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libbitlinear.so")
SOURCES = ["abi.hip", "pack.hip", "quant.hip", "gemv.hip", "gemm.hip", "backward.hip", "b3.hip"]
MEASURE_LIB_PATH = os.path.join(HERE, "libblmeasure.so")
MEASURE_SOURCES = ["measure.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # IEEE fp32 division (the ternarization and the activation scale are
    # defined with correctly rounded fp32 division) and no FMA contraction
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into SGPRs by the dispatcher: the first
    # instructions need no scalar load round trip (a decode launch is a
    # latency chain of a few microseconds)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
]


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def kernel_resources(compiler_output: str) -> dict:
    """Per-kernel resource usage from the compiler's resource remarks:
    {mangled name: {"VGPRs": .., "AGPRs": .., "ScratchSize [bytes/lane]": .., ...}}."""
    kernels, current = {}, None
    for ln in compiler_output.splitlines():
        if "remark:" not in ln:
            continue
        body = ln.split("remark:", 1)[1].split("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            current = body.split(":", 1)[1].strip()
            kernels[current] = {}
        elif current and ":" in body:
            key, val = body.rsplit(":", 1)
            kernels[current][key.strip()] = val.strip()
    return kernels


def _build_lib(sources, lib_path, tmp, verbose):
    """Compile `sources` in parallel and link them into `lib_path`.  Every
    kernel must run from registers: a kernel with scratch memory (a spill, or
    a register array indexed at run time) fails the build."""
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, RESOURCE_REMARKS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed, scratch = [], []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "remark:" not in ln
                 and "kernel-resource-usage" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines))
        if p.returncode:
            failed.append(src)
            continue
        for name, res in kernel_resources(out).items():
            if verbose:
                print(f"{src}: {name}: VGPRs {res.get('VGPRs')} AGPRs {res.get('AGPRs')} "
                      f"scratch {res.get('ScratchSize [bytes/lane]')} LDS {res.get('LDS Size [bytes/block]')}")
            if res.get("ScratchSize [bytes/lane]", "0") != "0":
                scratch.append(f"{src}: {name} ({res['ScratchSize [bytes/lane]']} bytes/lane)")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    if scratch:
        raise RuntimeError("kernels using scratch memory: " + "; ".join(scratch))
    tmp_lib = lib_path + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp_lib],
                   check=True)
    os.replace(tmp_lib, lib_path)


def build(verbose: bool = False) -> str:
    """Build both libraries; returns the path of libbitlinear.so."""
    with tempfile.TemporaryDirectory(prefix="bitlinear_build_") as tmp:
        _build_lib(SOURCES, LIB_PATH, tmp, verbose)
        _build_lib(MEASURE_SOURCES, MEASURE_LIB_PATH, tmp, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
