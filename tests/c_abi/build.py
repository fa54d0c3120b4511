"""Build tests/c_abi/kda_c_consumer: a plain C++ caller of include/kda.h,
linked against libkda.so and, as its checker, the oracle's library (both
found next to the binary's tree through its run path)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "kda_c_consumer")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build():
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "kda_c_consumer.cpp"),
           "-L", os.path.join(ROOT, "gated_delta_rule_23_amd"), "-l:libkda.so",
           "-L", os.path.join(ROOT, "oracle"), "-l:libkda_oracle.so",
           "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_23_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-o", BIN + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)


if __name__ == "__main__":
    build()
