"""Build the seeded input generator: synth/libsynth.so (host, gcc) and synth/libsynth_dev.so (the
device-side cache filler, hipcc for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_dev(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", DEV_LIB + ".tmp", os.path.join(HERE, "synth_dev.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for synth_dev.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(DEV_LIB + ".tmp", DEV_LIB)
    return DEV_LIB


def build(verbose: bool = False, device: bool = True) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", LIB + ".tmp",
           os.path.join(HERE, "synth.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    if device:
        build_dev(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
