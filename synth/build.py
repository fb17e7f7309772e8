"""Builds the seeded input generator: a host library (gcc) and its device twin (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
GPU_LIB = os.path.join(HERE, "libsynth_gpu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> None:
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-std=c11", "-fPIC", "-shared", "-Wall", "-o", HOST_LIB + ".tmp",
         os.path.join(HERE, "gen.c")],
        [HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", GPU_LIB + ".tmp", os.path.join(HERE, "gen_gpu.hip")],
    ]
    for cmd, out in zip(cmds, (HOST_LIB, GPU_LIB)):
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose=True)
