"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

* The C oracle, built by gcc with -fsanitize=address,undefined (abort on the
  first report), runs its pin tests.
* The host side of libgdla.so -- every argument check of the C ABI -- built
  with the same sanitizers on its host pass only (the gfx950 device code is
  not instrumented), runs the boundary tests, whose rejected calls launch
  nothing.

Each run is a child process with the sanitizer runtime preloaded (python
itself is not instrumented); leak checking is off, since the interpreter
keeps its allocations to the end.  Skipped where a runtime or compiler is
missing.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _gcc_asan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _run_child(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return tail


def test_oracle_pins_under_sanitizers(tmp_path):
    preload = _gcc_asan()
    if preload is None:
        pytest.skip("gcc's AddressSanitizer runtime not found")
    from oracle import build
    lib = build.build_oracle(out=str(tmp_path / "liboracle_san.so"), extra=SAN)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle; oracle._LIB = oracle._bind(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r, '-k', 'not mutant']))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    out = _run_child(code, preload)
    assert " passed" in out


def test_host_checks_under_sanitizers(tmp_path):
    preload = _clang_asan()
    if preload is None:
        pytest.skip("the ROCm compiler's AddressSanitizer runtime not found")
    from attention_gdla_prefill_amd import build
    flags = []
    for f in SAN:                       # host pass only
        flags += ["-Xarch_host", f]
    lib = build.build_library(extra_flags=flags, out=str(tmp_path / "libgdla_san.so"), quiet=True)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import attention_gdla_prefill_amd._lib as L\n"
            "L._lib = L.load(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_boundary.py")))
    out = _run_child(code, preload)
    assert " passed" in out
