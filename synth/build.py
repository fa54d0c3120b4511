"""Build the synthetic-input generator: a host library (gcc) and a device
library (hipcc, gfx950). Floating-point contraction is off on both so the
two produce identical bits."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(HERE, "libsynth_device.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    subprocess.run(cmd, check=True)


def build(device=True):
    _run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
          "-I", CSRC, os.path.join(CSRC, "synth_host.c"), "-o", HOST_LIB + ".tmp"])
    os.replace(HOST_LIB + ".tmp", HOST_LIB)
    if device:
        _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", CSRC, os.path.join(CSRC, "synth_device.hip"), "-o", DEVICE_LIB + ".tmp"])
        os.replace(DEVICE_LIB + ".tmp", DEVICE_LIB)


if __name__ == "__main__":
    build()
