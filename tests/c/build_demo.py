"""Compile tests/c/bsg_forward_demo.c, a plain C caller of libbsg.so (gcc,
linked against the in-tree libbsg.so and the HIP runtime)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "bsg_forward_demo.c")
EXE = os.path.join(HERE, "bsg_forward_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "block_sparse_gemm_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-L", pkg, "-lbsg", "-Wl,-rpath,$ORIGIN/../../block_sparse_gemm_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-o", EXE + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
