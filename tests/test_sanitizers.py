"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle is compiled with -fsanitize=address,undefined (every report fatal) and every pin runs
  against that copy, in a child Python process with the sanitizer runtime preloaded (the interpreter
  itself is not instrumented).  The pins include the NaN-reach causality check, so out-of-bounds or
  uninitialised reads in the recurrences would show here.
* The plain C99 consumer of include/la2.h is compiled the same way and run against the built
  library: the ABI's argument checks and status strings, called from sanitized C.
"""
import os
import shutil
import subprocess
import sys

import pytest

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import binding
from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
orc = oracle.load({lib!r})
for pin in pins.ALL_PINS:
    pin(orc)
    print("pin ok", pin.__name__, flush=True)
print("ALL PINS OK", len(pins.ALL_PINS))
"""


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    lib = obuild.compile_oracle(obuild.SRC, str(tmp_path / "liboracle_san.so"), extra_flags=SAN)
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="4", **ENV_SAN)
    run = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=TESTS, lib=lib)], env=env,
                         capture_output=True, text=True, timeout=900)
    print(run.stdout[-2000:], run.stderr[-4000:])
    assert run.returncode == 0, run.stderr[-4000:]
    assert "ALL PINS OK" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr


PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "la2.h"

int main(void) {
    int bad = 0;
    for (int s = 0; s <= 9; ++s)
        if (la2_status_string(s) == NULL || strlen(la2_status_string(s)) == 0) bad = 1;
    /* rejected before anything is enqueued: NULL pointers, bad sizes, unsupported head size and tile */
    int st = la2_forward(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 64, 64, 64, LA2_BF16, NULL, 0, NULL);
    if (st != LA2_ERR_NULL_POINTER) bad = 2;
    st = la2_forward((void *)0x100000, (void *)0x200000, (void *)0x300000, NULL, (void *)0x400000,
                     1, 1, 0, 64, 64, 64, LA2_BF16, NULL, 0, NULL);
    if (st != LA2_ERR_BAD_SHAPE) bad = 3;
    st = la2_backward((void *)0x100000, (void *)0x200000, (void *)0x300000, NULL, (void *)0x400000,
                      (void *)0x500000, (void *)0x600000, (void *)0x700000, 1, 1, 64, 64, 64, 100, LA2_F32,
                      NULL, 0, NULL);
    if (st != LA2_ERR_UNSUPPORTED) bad = 4;
    /* a split chain without its workspace */
    st = la2_forward((void *)0x1000000, (void *)0x2000000, (void *)0x3000000, NULL, (void *)0x4000000,
                     1, 1, 4096, 128, 128, 128, LA2_BF16, NULL, 0, NULL);
    if (st != LA2_ERR_WORKSPACE_TOO_SMALL) bad = 5;
    for (int b = 16; b <= 256; b *= 2)
        if (la2_workspace_bytes(1, 16, 131072, 128, 128, b, LA2_BF16, 1) == (size_t)-1 ||
            la2_workspace_bytes(1, 16, 131072, 128, 128, b, LA2_F32, 1) == (size_t)-1) bad = 6;
    if (la2_workspace_bytes(1, 1, 64, 96, 64, 64, LA2_BF16, 0) != (size_t)-1) bad = 7;
    printf("abi %d bad %d\n", la2_abi_version(), bad);
    return bad;
}
"""


def test_plain_c_consumer_under_asan_ubsan(tmp_path):
    if _runtime("libasan.so") is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    la2.load_library()
    src = tmp_path / "use_la2.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_la2"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, f"-I{os.path.join(ROOT, 'include')}",
                    str(src), f"-L{libdir}", "-lla2", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True,
                   capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=dict(os.environ, **ENV_SAN))
    print(run.stdout, run.stderr[-4000:])
    assert run.returncode == 0, run.stderr[-4000:]
    assert f"abi {binding.LA2_ABI_VERSION} bad 0" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr


def test_sanitizer_harness_reports_a_planted_overflow(tmp_path):
    """The harness is not vacuous: a copy of the oracle that reads one element past its state buffer
    fails under the same run."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    src = open(obuild.SRC).read()
    old = "acc += S[i * dv + j] * qt[i];"
    assert src.count(old) == 1
    bad = tmp_path / "oracle_overflow.c"
    bad.write_text(src.replace(old, "acc += S[i * dv + j + (i == d - 1 && j == dv - 1)] * qt[i];"))
    lib = obuild.compile_oracle(str(bad), str(tmp_path / "liboracle_bad.so"), extra_flags=SAN)
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="2", **ENV_SAN)
    run = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=TESTS, lib=lib)], env=env,
                         capture_output=True, text=True, timeout=300)
    assert run.returncode != 0
    assert "heap-buffer-overflow" in run.stderr
