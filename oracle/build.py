"""Build the CPU oracle (oracle.c, kvcache.c -> liboracle.so) with gcc.

Test infrastructure: the library is loaded only by the tests, the smoke check
and the benchmark's cpu_baseline leg.  Binary32 arithmetic must be plain IEEE:
no contraction into fused multiply-adds and no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "kvcache.c")]
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-frounding-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
