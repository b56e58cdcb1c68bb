"""Sanitizer run on the CPU: the oracle and the host side of the C ABI
(argument validation and launch planning, api.cpp and plan.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc; every report is fatal),
then driven by the existing host-side tests in a process with the sanitizer
runtimes preloaded: the oracle's pins (hand cases, golden files, closed
forms, codebooks, brute force) and exact encoder boundary cases through the
instrumented oracle, the ABI's validation cases and every seeded random KV
and QK case through the instrumented host layer, whose launchers are stubs
that check the plan and launch nothing (tests/sanitize/).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qk_rmsnorm_rope_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


def test_oracle_and_host_abi_under_asan_and_ubsan(tmp_path):
    oracle_lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"] + SAN +
                   [os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_lib, "-lm"], check=True)
    host_lib = str(tmp_path / "libqknr_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN +
                   [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
                    "-o", host_lib, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    # reports go to files: pytest's capture of fd 2 inside the child would
    # swallow a report printed just before the sanitizer ends the process
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
               ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan",
               QKNR_ORACLE_LIB=oracle_lib, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "run_host_cases.py"), host_lib],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    reports = "".join(p.read_text()[-3000:] for p in sorted(logs.iterdir()))
    out = r.stdout[-3000:] + r.stderr[-2000:] + reports
    assert not reports, out
    assert r.returncode == 0, out
    assert "full entry-point calls: 0 unexpected statuses" in r.stdout, out
