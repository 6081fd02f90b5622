"""The oracle's pins once more, with oracle.c built under AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only): every out-of-bounds access, use of freed
memory, signed overflow, bad shift or misaligned load in the checker fails the run.

The instrumented library is loaded into a child interpreter through FP8KV_ORACLE_LIB, with
the ASan runtime preloaded ahead of whatever the environment already preloads (a shared
library built with ASan needs its runtime first in the process).  Leak checking is off: the
interpreter itself keeps allocations alive at exit.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_codec.py", "test_oracle_codecs.py", "test_oracle_attention.py",
             "test_oracle_per_head.py", "test_oracle_prefill.py", "test_oracle_rotation.py"]
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _runtime(name: str) -> str:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                       check=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else ""


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = str(tmp_path / "liboracle_san.so")
    flags = [f for f in oracle.GCC_FLAGS if not f.startswith("-O")]
    subprocess.check_call(["gcc", *flags, *SAN_FLAGS, oracle._SRC, "-o", lib, "-lm"])
    env = dict(os.environ)
    env["FP8KV_ORACLE_LIB"] = lib
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    # -s: a sanitizer report goes straight to stderr (pytest's capture would drop it when the
    # runtime ends the process inside a test)
    cmd = [sys.executable, "-m", "pytest", "-s", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
