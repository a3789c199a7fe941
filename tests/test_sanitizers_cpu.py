"""Host sanitizers: the oracle's pins and the library's host-side argument
checks under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

* The oracle (kda_oracle.c) is built with gcc -fsanitize=address,undefined
  and the oracle pin tests run against it in a child process that starts with
  gcc's ASan/UBSan runtimes preloaded.
* The library is built with the sanitizers on its host code (hipcc
  -Xarch_host -fsanitize=...; the device code is built as usual) and the C ABI
  validation tests run against it in a child process that starts with clang's
  ASan runtime preloaded.  No GPU is touched: those tests exercise the checks
  that run before any launch.

Every sanitizer report is fatal (-fno-sanitize-recover=all), so a report fails
the child's pytest run; the output is also scanned for report headers.
Leak checking is off: the Python interpreter itself does not free everything
at exit.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehaviorSanitizer")


def _gcc_runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _run_pytest(files, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"] + files
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    for rep in REPORTS:
        assert rep not in text, text[-4000:]
    return text


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    from oracle.oracle import build_oracle_sanitized
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    so = build_oracle_sanitized(str(tmp_path / "libkda_oracle_san.so"))
    text = _run_pytest(["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py"],
                       {"LD_PRELOAD": asan + ":" + ubsan, "KDA_ORACLE_LIBRARY": so}, timeout=900)
    assert " passed" in text


def test_abi_checks_under_asan_ubsan(tmp_path):
    from gated_delta_rule_66_amd import build as B
    try:
        B.hipcc()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    so = B.build_library_sanitized(str(tmp_path / "libkda_san.so"))
    text = _run_pytest(["tests/test_abi_cpu.py"], {"LD_PRELOAD": rt, "KDA_LIBRARY": so}, timeout=900)
    assert " passed" in text
