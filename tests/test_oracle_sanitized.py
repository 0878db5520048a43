"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is built with gcc's address and undefined-behaviour sanitizers into a temporary
library, and the pin tests run against it in a subprocess with the ASan runtime preloaded
(leak detection off: the interpreter's own allocations are not the oracle's). Any sanitizer
report aborts the run. A control copy with one planted out-of-bounds write must be reported,
so a run that passes shows the sanitizers were live. The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# the control: orc_topk's scored copy written one element past its end
PLANT_ORIG = "for (int j = 0; j < n; ++j) { v[j].s = s[j]; v[j].j = j; }"
PLANT_BAD = "for (int j = 0; j <= n; ++j) { v[j].s = s[j]; v[j].j = j; }"


def _runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(src_text, tmp_path, tag):
    c_file = tmp_path / ("oracle_%s.c" % tag)
    c_file.write_text(src_text)
    lib = tmp_path / ("liboracle_%s.so" % tag)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", str(c_file), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    return lib


def _run_pins(lib, asan, log_dir):
    """Runs the pins against lib; returns (the run, the text of every sanitizer report). Reports
    go to files under log_dir, since the inner pytest captures the process's stderr."""
    log_dir.mkdir()
    env = dict(os.environ, MSA_ORACLE_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:log_path=%s" % (log_dir / "asan"),
               UBSAN_OPTIONS="print_stacktrace=1:log_path=%s" % (log_dir / "ubsan"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    reports = "".join(p.read_text() for p in sorted(log_dir.iterdir()))
    return r, reports


@pytest.mark.slow
def test_pins_clean_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(SRC).read()
    lib = _build(src, tmp_path, "san")
    r, reports = _run_pins(lib, asan, tmp_path / "logs")
    assert reports == "", reports[-3000:]
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]

    assert src.count(PLANT_ORIG) == 1
    bad = _build(src.replace(PLANT_ORIG, PLANT_BAD), tmp_path, "san_control")
    rc, reports = _run_pins(bad, asan, tmp_path / "logs_control")
    assert rc.returncode != 0 and "heap-buffer-overflow" in reports, \
        "the planted out-of-bounds write was not reported:\n" + reports[-2000:]
