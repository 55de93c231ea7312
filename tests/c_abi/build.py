"""Build tests/c_abi/run_from_c, the C99 program that drives the library on
the GPU through the HIP runtime's C API and include/skinny.h (host code only:
gcc, no device compiler).  Called by __graft_entry__.build(); the GPU test
that runs the program does not build it."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "run_from_c")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.join(ROOT, "skinny_bf16_decode_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "run_from_c.c"), "-o", EXE,
           "-L", lib_dir, "-lskinny", "-Wl,-rpath,$ORIGIN/../../skinny_bf16_decode_amd",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
