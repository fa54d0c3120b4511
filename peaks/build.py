"""Build libpeaks.so: the copy and MFMA micro-benchmarks (gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build():
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(HERE, "peaks.hip"), "-o", LIB + ".tmp"], check=True)
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build()
