"""Builds tests/c/fa2_c_client (a plain C program using include/fa2.h) with gcc,
linked against the in-tree libfa2.so and the CPU oracle library.

    python tests/c/build_client.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "fa2_c_client")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra",
           # the HIP runtime's C header needs its platform named
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "fa2_c_client.c"),
           "-L", os.path.join(ROOT, "exact_attention_23_amd"), "-l:libfa2.so",
           "-L", os.path.join(ROOT, "oracle"), "-l:libfa2_oracle.so",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../exact_attention_23_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
