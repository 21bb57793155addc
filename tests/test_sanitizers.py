"""Host-side sanitizer run: the C ABI's argument checks and workspace layout
(``muse_attn.cpp``) and the CPU oracle (``oracle.c``), each built with
AddressSanitizer and UndefinedBehaviorSanitizer, under the ABI tests and the
oracle pins.  GPU code is not instrumented (the GPU has no sanitizer here);
these tests make no GPU call.  The child process preloads clang's ASan
runtime, since the Python interpreter itself is not instrumented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_oracle_pins_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from full_gqa_attention_amd import build as fa_build
    import oracle
    fa_build.build_sanitized()
    oracle.build_sanitized()
    env = dict(os.environ)
    env.update({
        "MUSE_SANITIZED": "1",
        "LD_PRELOAD": fa_build.asan_runtime(),
        # the interpreter and the HIP runtime are not instrumented: their
        # allocations stay outside the leak check
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=900)
    out = r.stdout.decode(errors="replace")
    tail = "\n".join(out.splitlines()[-40:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, tail
    assert "sanitized library libmuse_attn_san.so loaded: True" in out, tail
    assert "sanitized library liboracle_san.so loaded: True" in out, tail
