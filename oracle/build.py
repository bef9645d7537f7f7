"""Build the CPU oracle (plain C, one thread).

-ffp-contract=off: no multiply-add fusion anywhere (OPEN-1B paper, section
2.1, "Fused multiply-add").  -fno-fast-math keeps IEEE semantics;
-fno-math-errno lets sqrtf become the correctly rounded SSE instruction;
-frounding-math stops build-time folding, since the oracle's operations run
under a run-time FTZ/DAZ mode.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "repro_oracle.c")
LIB = os.path.join(HERE, "librepro_oracle.so")
FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-fno-math-errno", "-frounding-math", "-mfpmath=sse", "-msse2"]


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    cmd = ["gcc", *FLAGS, *extra, SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
