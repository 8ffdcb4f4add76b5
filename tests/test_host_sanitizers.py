"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The C++ oracle, built with g++ ``-fsanitize=address,undefined``, runs the
  oracle pins and the numpy cross-check in a child process that preloads the
  sanitizer runtime.
* The library's host code (argument checks, step planning, workspace sizing,
  the describe call the cost model reads), built with hipcc with the
  sanitizers on the host side only (device code is compiled as usual and not
  run), runs the host ABI tests and the cost-model tests the same way.

A sanitizer report ends the child with an error, so the test fails (the child
runs pytest without output capture, so the report reaches its stderr).  A
control run on a copy of the oracle with a planted one-past-the-end read must
end in a report.  The child keeps any preload the environment already has,
after the runtime.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",  # the interpreter itself leaks by design
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "PYTHONDONTWRITEBYTECODE": "1"}


def _runtime(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _child(preload, code, timeout=600):
    env = dict(os.environ, **SAN_ENV)
    env["LD_PRELOAD"] = ":".join(p for p in (preload, os.environ.get("LD_PRELOAD", "")) if p)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _oracle_san(tmp_path, name, plant=None):
    """Build oracle.cpp (optionally with one planted change) with the sanitizers
    and run the oracle pins and the cross-check on it in a child process."""
    gxx = shutil.which("g++")
    rt = _runtime([gxx, "-print-file-name=libasan.so"]) if gxx else None
    if rt is None:
        pytest.skip("g++ or its AddressSanitizer runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "oracle.cpp")).read()
    if plant is not None:
        assert src.count(plant[0]) == 1
        src = src.replace(*plant)
    cpp, lib = str(tmp_path / f"{name}.cpp"), str(tmp_path / f"lib{name}.so")
    open(cpp, "w").write(src)
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-fno-omit-frame-pointer", "-o", lib, cpp, "-lpthread"], check=True, capture_output=True)
    code = f"""
import sys
import oracle.cpp as C
C.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                      "tests/test_oracle_pins.py", "tests/test_oracle_cross.py"]))
"""
    return _child(rt, code)


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    r = _oracle_san(tmp_path, "oracle_san")
    assert r.returncode == 0 and "passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]


def test_sanitized_run_reports_a_planted_overread(tmp_path):
    """Control: the same run on a copy of the oracle whose top-k reads one score
    past the end of its input must end in an AddressSanitizer report."""
    r = _oracle_san(tmp_path, "oracle_overread",
                    ("for (int i = 0; i < C; ++i) v[i] = Scored{s[i], pages[i]};",
                     "for (int i = 0; i < C; ++i) v[i] = Scored{s[i + (i == C - 1)], pages[i]};"))
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.stdout[-1000:], r.stderr[-2000:])


def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    clang = "/opt/rocm/lib/llvm/bin/clang"
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    rt = _runtime([clang, "-print-file-name=libclang_rt.asan-x86_64.so"]) if os.path.exists(clang) else None
    if rt is None or not os.path.exists(hipcc):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    from free_sparse_attention_amd import build as fsa_build
    lib = str(tmp_path / "libfsa_hostsan.so")
    flags = [f for f in fsa_build.HIPCC_FLAGS if f != "-O3"]
    cmd = [hipcc, "-O1", "-g", *flags, "-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-o", lib, *fsa_build.sources()]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    code = f"""
import sys
from free_sparse_attention_amd import _lib
_lib.load({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                      "tests/test_abi_host.py", "tests/test_cost_model.py"]))
"""
    r = _child(rt, code)
    assert r.returncode == 0 and "passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
