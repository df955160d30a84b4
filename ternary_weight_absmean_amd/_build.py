"""Build ``libbitlinear.so`` (the C-ABI HIP library) for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libbitlinear.so")
SOURCES = ["abi.hip", "pack.hip", "quant.hip", "gemv.hip", "gemm.hip"]

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


def build(verbose: bool = False) -> str:
    """Compile every HIP source in parallel and link the shared library."""
    with tempfile.TemporaryDirectory(prefix="bitlinear_build_") as tmp:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines))
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB_PATH + ".tmp"
        subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], check=True)
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
