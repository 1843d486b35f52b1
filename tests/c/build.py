"""Build tests/c/abi_driver: a C++ program that uses libmoedc through its C
ABI only (linked against the in-tree libmoedc.so, found through an rpath
relative to the executable)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "combine_moedc_route_amd")
SRC = os.path.join(HERE, "abi_driver.cpp")
EXE = os.path.join(HERE, "_build", "abi_driver")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    rel = os.path.relpath(PKG, os.path.dirname(EXE))
    cmd = [HIPCC, "-O2", "-std=c++17", "-Wall", "-Werror", "-I" + os.path.join(ROOT, "include"),
           SRC, "-o", EXE + ".tmp", "-L" + PKG, "-lmoedc", "-Wl,-rpath,$ORIGIN/" + rel]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the ABI driver failed:\n{r.stdout}\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
