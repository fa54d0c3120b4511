"""Build the fp64 CPU oracle (plain C, gcc).  Test infrastructure only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkda_oracle.so")


def build():
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", os.path.join(HERE, "kda_oracle.c"),
                    "-lm", "-o", LIB + ".tmp"], check=True)
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build()
