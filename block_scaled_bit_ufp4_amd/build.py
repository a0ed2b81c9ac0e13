"""Build libufp4.so (the HIP library) in-tree with hipcc for gfx950.

Flags: -ffp-contract=off (no fused multiply-adds the definitions do not
write), fp32 denormals kept, correctly rounded binary32 division (hipcc's
default), packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libufp4.so")
SOURCES = ["api.hip", "quantize.hip", "dequant_stats.hip", "gemm.hip", "kvdecode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    objs = []
    procs = []
    for s in SOURCES:
        obj = os.path.join(CSRC, s.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj]
        objs.append(obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(procs):
    err = None
    while procs:
        p = procs.pop(0)
        _, stderr = p.communicate()
        lines = [ln for ln in (stderr or "").splitlines()
                 if "packed-fp32-ops" not in ln and "unknown target feature" not in ln and ln.strip()]
        if p.returncode != 0:
            err = "\n".join(lines)
        elif lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if err:
        raise RuntimeError("hipcc failed:\n" + err)


if __name__ == "__main__":
    print(build(verbose=True))
