"""The library's host code (plan creation, validation, sizing, workspace
layout and the kernel arguments of every C entry point), the host planners
and the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
tests/c/sanitize_host.cpp links host.cpp and planning.cpp against stand-in
launchers that check every argument a kernel would receive, and a copy
stand-in that really copies the table image into host memory playing the
workspace; it drives random valid and invalid layer descriptions and calls,
random planner inputs and random small layers through every oracle
function.  Built with g++ (host code only; no GPU code is compiled)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_moedc_route_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc/g++")
def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    inc = ["-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in (os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "planning.cpp"),
                os.path.join(ROOT, "tests", "c", "sanitize_host.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["g++", "-std=c++17", "-O1", "-g", *san, *inc, "-c", src, "-o", o],
                       check=True)
        objs.append(o)
    o = str(tmp_path / "moedc_oracle.o")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", *san, "-c",
                    os.path.join(ROOT, "oracle", "moedc_oracle.c"), "-o", o], check=True)
    objs.append(o)
    exe = str(tmp_path / "sanitize_host")
    subprocess.run(["g++", *san, *objs, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitize_host ok" in r.stdout
    print(r.stdout.strip())
