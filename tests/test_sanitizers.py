"""Host sanitizers over the CPU code (no GPU): AddressSanitizer and
UndefinedBehaviorSanitizer builds of (1) the plain C oracle, run under its
pins, and (2) the C ABI's host code (argument checks, counts, workspace
sizes, the LVSA plan and the STA tile order), run under the ABI tests.

Each test builds its own copy in a temporary directory and runs the tests
in a child process with the sanitizer runtime preloaded (a shared library
built with ASan needs the runtime loaded first); any report ends the child
with a non-zero status.  Only host code is instrumented: the GPU code of
the ABI library is built as usual.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(args, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def asan_is_live(lib_path, preload, env_extra):
    """The child process really runs with the ASan runtime and the
    instrumented library (its ASan report hooks resolve)."""
    code = ("import ctypes, sys; ctypes.CDLL(%r); "
            "sys.exit(0 if hasattr(ctypes.CDLL(None), '__asan_report_load8') else 3)" % lib_path)
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    return subprocess.run([sys.executable, "-c", code], env=env, timeout=120).returncode == 0


@pytest.mark.timeout(900)
def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "libsla_oracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "sla_oracle.c"),
                           "-o", lib, "-lm"])
    preload = subprocess.check_output([gcc, "-print-file-name=libasan.so"], text=True).strip()
    assert asan_is_live(lib, preload, {})
    out = run_child(["-m", "pytest", "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py", "-x", "-q",
                     "-p", "no:cacheprovider"],
                    {"LD_PRELOAD": preload, "SLA_ORACLE_LIB": lib})
    assert " passed" in out


@pytest.mark.timeout(900)
def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    from sparse_attention_video_sla_amd import build
    build.build()                                        # the uninstrumented objects of the other sources
    obj = str(tmp_path / "api_san.o")
    # host-side instrumentation only: every -fsanitize= goes to the host pass
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-I" + os.path.join(ROOT, "include"),
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                           "-c", os.path.join(build.CSRC, "api.hip"), "-o", obj],
                          stderr=subprocess.DEVNULL)
    others = [os.path.join(build.BUILD, s.replace(".hip", ".o")) for s in build.SOURCES if s != "api.hip"]
    lib = str(tmp_path / "libsla_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           obj, *others, "-o", lib])
    preload = subprocess.check_output([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                      text=True, stderr=subprocess.DEVNULL).strip()
    if not os.path.isabs(preload) or not os.path.exists(preload):
        pytest.skip("clang ASan runtime not found")
    assert asan_is_live(lib, preload, {})
    out = run_child(["-m", "pytest", "tests/test_abi_cpu.py", "-x", "-q", "-p", "no:cacheprovider"],
                    {"LD_PRELOAD": preload, "SLA_TEST_LIB": lib})
    assert " passed" in out
