"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each exercised by the CPU tests that reach it, in a child process with the
matching ASan runtime preloaded:
  * the f64 oracle (gcc): the oracle pins;
  * the library's host code (hipcc, sanitizers on the host compilation only; the
    device code is built as usual): argument validation, the launch plan and its
    introspection, window segmentation, the binding's checks.
Any sanitizer report aborts the child and fails the test."""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.cpu
ROOT = Path(__file__).resolve().parent.parent


def _run_pytest(env_extra, tests, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", str(lib), str(ROOT / "oracle" / "mgattn_oracle.c"),
                    "-lm"], check=True)
    preload = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    _run_pytest({"MGATTN_ORACLE_LIB": str(lib)}, ["tests/test_oracle_pins.py", "-k", "not mutant"], preload)


def test_library_host_code_under_asan_ubsan(tmp_path):
    from vit_perception_encoder_amd import build as b

    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = tmp_path / "libmgattn_san.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g"]
    subprocess.run([hipcc, *b.COMMON, *b.DEVICE_FLAGS, *san, "-shared", "-o", str(lib), *map(str, b.SOURCES)],
                   check=True, capture_output=True)
    preload = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not Path(preload).exists():
        pytest.skip("clang ASan runtime not found")
    _run_pytest({"MGATTN_LIB": str(lib)},
                ["tests/test_boundary.py", "tests/test_window_host.py", "tests/test_binding_checks.py"], preload)
