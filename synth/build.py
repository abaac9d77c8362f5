"""Compile the synthetic-input fillers: synth/libsynth_cpu.so (gcc) and
synth/libsynth_gpu.so (hipcc, gfx950). Both include gen_core.h and are built with
-ffp-contract=off so that they produce identical bits."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(HERE, "libsynth_gpu.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> None:
    cmds = [
        (["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          os.path.join(HERE, "gen_cpu.c"), "-o", CPU_LIB + ".tmp", "-lm"], CPU_LIB),
        ([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          os.path.join(HERE, "gen_gpu.hip"), "-o", GPU_LIB + ".tmp"], GPU_LIB),
    ]
    for cmd, out in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose=True)
