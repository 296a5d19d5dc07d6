"""The oracle's pin suite on a copy of the oracle built with gcc's address and
undefined-behaviour sanitizers (CPU only).

zs_oracle.c is compiled a second time with ``-fsanitize=address,undefined``
(no recovery: the first finding aborts), then every pin of tests/pins.py runs
against that copy in a child Python process with the sanitizer runtime
preloaded.  An out-of-bounds access, use of freed memory, signed overflow,
misaligned access or other undefined behaviour anywhere the pins reach fails
the test; the pins' own value checks run as usual.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import oracle
import pins
o = oracle.Oracle({lib!r})
for pin in pins.ALL_PINS:
    pin(o)
    print("pin ok:", pin.__name__, flush=True)
print("all pins ok under the sanitizers", flush=True)
"""


def _runtime(name):
    path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's address-sanitizer runtime is not installed")
    lib = str(tmp_path / "libzs_oracle_san.so")
    flags = [f for f in oracle.GCC_FLAGS if f != "-O2"]
    subprocess.check_call(["gcc", *flags, "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           oracle._SRC, "-o", lib, "-lm"])
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    script = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, f"sanitized pin run failed ({r.returncode}):\n{r.stderr[-4000:]}"
    assert "all pins ok under the sanitizers" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
