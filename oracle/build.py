"""Build oracle/liboracle.so (test infrastructure) with gcc: scalar F32, no FP contraction."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *FLAGS, "-o", LIB + ".tmp", os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
