"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

oracle.c is built with both sanitizers (gcc, the same floating-point flags as
the regular build) and the whole pin suite (tests/test_oracle_pins.py) runs
against that build in a subprocess with the sanitizer runtime preloaded into
the Python process: every oracle function is called, at the pins' sizes and
special cases, with memory and undefined-behaviour checks on.  A copy with a
planted one-element over-write must make the same run fail with an
AddressSanitizer report that names the function, so the instrumentation is
known to be live.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(src_text, out):
    src = out.with_suffix(".c")
    src.write_text(src_text)
    subprocess.run(["gcc", *FLAGS, *SAN, "-o", str(out), str(src), "-lm"], check=True)
    return str(out)


def _run_pins(lib, asan, logdir):
    """The pin suite against `lib`; returns the run and the sanitizers' reports
    (written to files, since the test runner captures the process's stderr)."""
    log = os.path.join(str(logdir), "san")
    env = dict(os.environ, TPMLP_ORACLE_LIB=lib, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    reports = "".join(open(os.path.join(str(logdir), f)).read() for f in sorted(os.listdir(str(logdir)))
                      if f.startswith("san"))
    return r, reports


@pytest.fixture(scope="module")
def asan():
    path = _asan_runtime()
    if not path:
        pytest.skip("gcc's AddressSanitizer runtime not found")
    return path


def test_pins_pass_under_sanitizers(asan, tmp_path):
    lib = _build(open(SRC).read(), tmp_path / "liboracle_san.so")
    r, reports = _run_pins(lib, asan, tmp_path)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:] + reports[-3000:]
    assert reports == "", reports[-3000:]


def test_planted_over_write_is_reported(asan, tmp_path):
    """The fp64 reduction (the first function with this store) writes its last
    element one place past the end of Z."""
    text = open(SRC).read()
    old = "    Z[e] = acc;\n"
    assert text.count(old) >= 1
    new = "    Z[e + (e == n - 1)] = acc;\n"
    lib = _build(text.replace(old, new, 1), tmp_path / "liboracle_planted.so")
    r, reports = _run_pins(lib, asan, tmp_path)
    assert r.returncode != 0
    assert "AddressSanitizer" in reports and "oracle_partial_sum_f64" in reports, reports[-3000:]
