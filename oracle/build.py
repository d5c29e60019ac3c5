"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

Only the tests, the smoke check and the benchmark's cpu_baseline leg load the
result. Targets x86-64-v3 so the library built here also runs on other hosts.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["g++", "-O3", "-march=x86-64-v3", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wno-unknown-pragmas", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
