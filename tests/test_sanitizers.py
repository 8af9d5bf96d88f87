"""CPU sanitizer leg (rml "Quantization", section "Tests": the kernel tests also run
under AddressSanitizer and UndefinedBehaviorSanitizer).

Two host-side builds, each run in a child process with its sanitizer runtime
loaded first and any error fatal:
  - the C oracle built with gcc -fsanitize=address,undefined,float-cast-overflow
    (a float-to-int cast of an infinity is the kind of mistake the oracle once
    had), running every oracle pin and property test through it;
  - libqk.so with its host code (the C ABI's validation and dispatch) built with
    clang's AddressSanitizer and UndefinedBehaviorSanitizer (device code is built
    as usual), running the host-side ABI checks of test_capi_host.py.
Neither needs a GPU: no kernel is launched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(compiler, name):
    out = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found by {compiler}")
    return path


def _run_pytest(files, runtime, extra_env):
    env = dict(os.environ, **SAN_ENV, **extra_env)
    # the sanitizer runtime has to be the first library loaded into the process
    env["LD_PRELOAD"] = runtime + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in files]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
    return log


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    from oracle import build as oracle_build
    lib = str(tmp_path / "liboracle_san.so")
    oracle_build.build(["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
                        "-fno-sanitize-recover=all"], lib=lib)
    log = _run_pytest(["test_oracle_pins.py", "test_oracle_properties.py"], _runtime("gcc", "libasan.so"),
                      {"QK_ORACLE_LIB": lib})
    assert " passed" in log and "failed" not in log


def test_capi_host_code_under_asan_ubsan(tmp_path):
    from quantized_gemv_quantize_amd import build as qk_build
    clang = os.path.join(os.path.dirname(os.path.realpath(qk_build.hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    runtime = _runtime(clang, "libclang_rt.asan-x86_64.so")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    lib = str(tmp_path / "libqk.so")
    qk_build.build(extra=host_san, lib=lib, obj_dir=str(tmp_path / "obj"),
                   link_extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                               "-shared-libsan"])
    log = _run_pytest(["test_capi_host.py"], runtime, {"QK_LIB_PATH": lib})
    assert " passed" in log and "failed" not in log
