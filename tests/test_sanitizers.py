"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the oracle and the input generator (plain C), and the C ABI's argument checks
and workspace arithmetic (kvc_api.cpp, kvc_host.cpp, with the kernel launchers
replaced by no-op stand-ins), built with -fsanitize=address,undefined and
-fno-sanitize-recover=all, then driven over small inputs that reach every
function (tests/sanitize/driver.py). Any report aborts the run and fails the
test. No GPU code is built or run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_code_clean_under_sanitizers(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    orc = str(tmp_path / "liboracle_san.so")
    syn = str(tmp_path / "libsynth_san.so")
    api = str(tmp_path / "libkvc_api_san.so")
    run(["gcc", *SAN, "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-std=c11",
         os.path.join(ROOT, "oracle", "kvc_oracle.c"), "-o", orc, "-lm"])
    run(["gcc", *SAN, "-fopenmp", "-shared", "-fPIC", "-std=c11", os.path.join(ROOT, "synth", "synth.c"), "-o", syn,
         "-lm"])
    csrc = os.path.join(ROOT, "clustered_sparse_attention_kv_amd", "csrc")
    run(["g++", *SAN, "-shared", "-fPIC", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "kvc_api.cpp"),
         os.path.join(csrc, "kvc_host.cpp"), os.path.join(ROOT, "tests", "sanitize", "kvc_stubs.cpp"), "-o", api])
    env = dict(os.environ, LD_PRELOAD=libasan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "driver.py"), orc, syn, api],
                       capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "sanitized run clean" in r.stdout, report[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in report, report[-4000:]
