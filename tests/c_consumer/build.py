"""Build libd2f_consumer.so, the plain-C consumer of the C ABI that
tests/test_gpu_c_consumer.py loads: gcc (C99, host code only) against
include/d2f.h, the HIP runtime API and the in-tree libd2f.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libd2f_consumer.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "block_causal_attention_d2f_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROCM, "include"), os.path.join(HERE, "consumer.c"), "-o", LIB,
           "-L", pkg, "-ld2f", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../block_causal_attention_d2f_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C consumer failed:\n" + r.stdout + r.stderr)
    return LIB


if __name__ == "__main__":
    print(build())
