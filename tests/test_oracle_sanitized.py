"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle/oracle.c`` is compiled with ``-fsanitize=address,undefined`` (any
report is fatal) and ``tests/test_oracle_pins.py`` runs against that build
in a subprocess whose interpreter preloads the ASan runtime. A second build
with one planted out-of-bounds read must make that run fail with an ASan
report, which shows the sanitizers are live. CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             *[f for f in oracle.CFLAGS if f not in ("-O2",)]]
# a read one element past each activation row: past the array on the last row
OOB = ("acc += (double)bf16_bits_to_f32(x[i * k + j]) * (double)wrow[j];",
       "acc += (double)bf16_bits_to_f32(x[i * k + j + (j + 1 == k)]) * (double)wrow[j];")


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    # -s: a sanitizer report goes to the process's stderr, not to a test's capture
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _build(src_text, out, tmp_path):
    c = tmp_path / "oracle_san.c"
    c.write_text(src_text)
    subprocess.run(["gcc", *SAN_FLAGS, str(c), "-o", str(out), "-lm"], check=True)


@pytest.fixture(scope="module")
def asan():
    if _asan_runtime() is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return True


def test_pins_pass_under_asan_and_ubsan(asan, tmp_path):
    lib = tmp_path / "liboracle_san.so"
    _build(open(SRC).read(), lib, tmp_path)
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_planted_out_of_bounds_read_is_reported(asan, tmp_path):
    src = open(SRC).read()
    assert src.count(OOB[0]) == 1
    lib = tmp_path / "liboracle_oob.so"
    _build(src.replace(OOB[0], OOB[1]), lib, tmp_path)
    r = _run_pins(lib)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stderr[-3000:]
