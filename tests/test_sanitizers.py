"""Host-side sanitizer builds, run on the CPU.

The ABI layer's validation (``api.cpp``: every refusal returns before any HIP
call) and the fp64 oracle (``gdn_oracle.c``) are rebuilt with AddressSanitizer
and UndefinedBehaviorSanitizer, and the CPU tests that exercise them -- the ABI
checks and the oracle's pins -- run again, in a child process with the sanitizer
runtimes preloaded, against those builds.  Any sanitizer report fails the test.
The GPU kernels are not instrumented (their objects are linked as built)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_ssm_core_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "UndefinedBehaviorSanitizer")


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no %s here" % name)
    return os.path.realpath(path)


def _run_sanitized(args, env_extra, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = " ".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    # leak reports would list the interpreter's own allocations; stop on the first
    # error; reports go to files (pytest's capture of fd 2 would swallow a report
    # printed just before the process exits)
    rep = tmp_path / "report"
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=97:log_path=%s" % rep
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98:log_path=%s" % rep
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout + r.stderr
    reports = "".join(open(f).read() for f in sorted(glob.glob(str(rep) + "*")))
    assert not reports, reports[-4000:]
    for pat in REPORTS:
        assert pat not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in log, log[-4000:]
    return log


def test_abi_validation_under_asan_ubsan(tmp_path):
    """api.cpp built by g++ with ASan + UBSan, linked with the kernel objects of the
    regular build; the ABI tests (exports, struct layout, every refusal path)."""
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    if not objs:
        pytest.skip("the HIP objects are not built")
    api_o = tmp_path / "api.o"
    lib = tmp_path / "libgdn_sanitized.so"
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")] + SAN
                   + ["-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", str(api_o)], check=True)
    subprocess.run(["g++", "-shared", "-fPIC"] + SAN[:1] + [str(api_o)] + objs
                   + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)], check=True)
    _run_sanitized(["tests/test_abi.py"], {"GDN_LIBRARY": str(lib)}, tmp_path)


def test_oracle_under_asan_ubsan(tmp_path):
    """gdn_oracle.c built by gcc with ASan + UBSan (and OpenMP); the oracle's pins."""
    lib = tmp_path / "liboracle_sanitized.so"
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math"] + SAN
                   + [os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", str(lib), "-lm"], check=True)
    _run_sanitized(["tests/test_oracle_pins.py", "tests/test_oracle_pins_variants.py", "tests/test_oracle_golden.py"],
                   {"GDN_ORACLE_LIBRARY": str(lib)}, tmp_path)
