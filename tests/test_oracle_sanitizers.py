"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C oracle is rebuilt with -fsanitize=address,undefined (every report fatal)
and the whole pin suite runs against that build; a second build with one planted
heap overflow must be stopped by the sanitizer, which shows that the net is live.
The sanitizer runtime is preloaded into the child Python process only, and only
where nothing else is preloaded (it must come first in the library list)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import ckv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]


def _runtime(name: str) -> str:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else ""


def _env_or_skip(lib: str) -> dict:
    if os.environ.get("LD_PRELOAD") or os.path.exists("/etc/ld.so.preload"):
        pytest.skip("another library is preloaded; the sanitizer runtime must come first")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    return dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
                UBSAN_OPTIONS="print_stacktrace=1", CKV_ORACLE_LIB=lib)


def _build(src_text: str, tmp_path) -> str:
    src = tmp_path / "oracle_san.c"
    src.write_text(src_text)
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *SAN_FLAGS, str(src), "-o", str(so), "-lm"])
    return str(so)


def _pins(env, *extra):
    # -s: a sanitizer report aborts the process, so it must not sit in pytest's capture
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py"), *extra],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)


def test_pin_suite_clean_under_asan_and_ubsan(tmp_path):
    env = _env_or_skip(_build(open(O.SRC).read(), tmp_path))
    r = _pins(env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_sanitizer_stops_a_planted_heap_overflow(tmp_path):
    """ckvo_attend's logit buffer one element short: the last logit is written past
    the allocation, which the fp64 results may not reveal but ASan must."""
    src = open(O.SRC).read()
    old = "double *z = (double *)malloc(sizeof(double) * (size_t)len);"
    assert src.count(old) == 1
    env = _env_or_skip(_build(src.replace(old, old.replace("(size_t)len", "(size_t)(len - 1)")),
                              tmp_path))
    r = _pins(env, "-k", "attend")
    assert r.returncode != 0 and "heap-buffer-overflow" in (r.stdout + r.stderr)
