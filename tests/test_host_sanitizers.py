"""Host AddressSanitizer and UBSan builds of the planner and the C oracle.

Both are plain host code, so each is compiled here with the host compilers
(g++ for the planner, gcc for the oracle) under -fsanitize=address,undefined
with every report fatal, and driven over random problems:

* tests/host_sanitize/plan_stress.cpp: valid and corrupted problems through
  the planner, the plan export (too small a buffer, then exact), the workspace
  size and the largest unit, checking that every accepted plan's units
  partition each request's streamed pages.  Leak detection stays on, so a plan
  that destroy does not free fails.
* tests/host_sanitize/oracle_stress.c: random small problems in every KV
  format, full and sampled rows, key ranges and sliding windows, inputs the
  oracle must reject, and the element decoders over every code.

No GPU code is built: the HIP sources never see a sanitizer flag.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _compile(cmd, tmp_path):
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=300)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower():
        pytest.skip("host sanitizer runtime not available: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr[-3000:]


def _run(exe, args, env_extra):
    env = dict(os.environ, **env_extra)
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    if res.returncode != 0 and "does not come first" in res.stderr:
        pytest.skip("another preloaded library keeps the sanitizer runtime from starting")
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    return res.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_stress")
    _compile(["g++", "-std=c++17", *SAN, "-I", "include",
              "-I", os.path.join("speculative_decode_verify_sweep_amd", "csrc"),
              os.path.join(HERE, "plan_stress.cpp"),
              os.path.join("speculative_decode_verify_sweep_amd", "csrc", "plan.cpp"),
              "-o", exe], tmp_path)
    out = _run(exe, ["3000"], {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                               "UBSAN_OPTIONS": "print_stacktrace=1"})
    accepted, rejected = [int(x) for x in out.split(":")[1].replace(",", " ").split()[::2]]
    assert accepted + rejected == 3000
    assert accepted > 1000 and rejected > 300, out     # both kinds really exercised


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_stress")
    _compile(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(HERE, "oracle_stress.c"),
              os.path.join("oracle", "attention.c"), "-o", exe, "-lm"], tmp_path)
    # leak checking is off here: OpenMP's runtime keeps its thread pool's
    # allocations until exit, which LeakSanitizer would report
    out = _run(exe, ["300"], {"ASAN_OPTIONS": "detect_leaks=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1",
                              "OMP_NUM_THREADS": "4"})
    assert "300 problems, ok" in out, out
