"""Build libmoedc.so (HIP kernels + C ABI) for gfx950, in-tree.

Every translation unit is compiled by hipcc for gfx950 only, with IEEE fp32
semantics (no fast-math, no FMA contraction, correctly rounded division,
denormals kept) and with packed-fp32 instruction selection disabled.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoedc.so")
# Measurement kernels for the benchmark's bandwidth ceilings (not the MoE path).
CEILING_LIB = os.path.join(HERE, "libmoedc_ceiling.so")
# The same library with dispatch's per-wave phase stamps (MOEDC_TRACE).
TRACE_LIB = os.path.join(HERE, "libmoedc_trace.so")
SOURCES = ["route.hip", "dispatch.hip", "fused.hip", "combine.hip", "stub.hip",
           "expert_gemm.hip", "noalloc.hip", "host.cpp", "planning.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src, verbose, defines=(), tag=""):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *CFLAGS, *["-D" + d for d in defines], *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, verbose):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_in = [(s, (), "") for s in SOURCES + ["ceiling.hip"]]
    jobs_in.append(("dispatch.hip", ("MOEDC_TRACE",), "_trace"))
    jobs = min(len(jobs_in), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        built = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs_in))
    objs = {(s, tag): o for (s, _, tag), o in zip(jobs_in, built)}
    _link([objs[(s, "")] for s in SOURCES], LIB, verbose)
    _link([objs[("ceiling.hip", "")]], CEILING_LIB, verbose)
    _link([objs[(s, "_trace" if s == "dispatch.hip" else "")] for s in SOURCES], TRACE_LIB,
          verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
