"""Build libkda.so: the C ABI of include/kda.h and its gfx950 kernels."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_prefill_bf16.hip", "kda_epilogue.hip",
           "kda_compose.hip", "kda_split.hip"]

# Packed fp32 VALU forms are kept out of the device code; the host pass does
# not know the feature and says so, which is harmless.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(extra_flags=()):
    srcs = []
    for s in SOURCES:
        srcs += (["-x", "hip"] if s.endswith(".cpp") else []) + [os.path.join(CSRC, s)]
    cmd = [HIPCC] + FLAGS + list(extra_flags) + srcs + ["-o", LIB + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build()
