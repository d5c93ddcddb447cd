"""Build the HIP library ``causal_linear_attention_amd/lib/libla2.so`` for gfx950.

Every source is compiled by hipcc for gfx950 only; objects go to ``_build/``
(not committed) and are linked into one shared library with a plain C ABI
(``include/la2.h``).  A second library, ``lib/libla2_testhooks.so``, links the
same kernel objects with the C ABI compiled under ``LA2_TEST_HOOKS`` and a plain
HBM stream kernel: it also exports ``la2_test_set_plan``, through which the tests
force work decompositions, and ``la2_test_stream``, which ``bench.py --stream``
times (``include/la2_test_hooks.h``).  Nothing else loads it.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libla2.so")
TEST_LIB = os.path.join(LIBDIR, "libla2_testhooks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["la2_scan_bf16.hip", "la2_fwd1_bf16.hip", "la2_bwd1_bf16.hip", "la2_state_bf16.hip", "la2_dkdv_bf16.hip", "la2_scan_f32.hip", "la2_prefix.hip", "la2_decode.hip", "la2_norm.hip",
           "la2_serial.hip", "la2_api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src, extra=(), tag=""):
    obj = os.path.join(OBJDIR, os.path.basename(src) + tag + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def _link(objs, out):
    tmp = out + ".tmp"
    # -Bsymbolic: each library calls its own internal functions, whichever other copy is loaded
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-Bsymbolic", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build_library(verbose=False, extra=()):
    """Compile every source and link ``libla2.so`` and ``libla2_testhooks.so``; returns the release path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = ([(s, tuple(extra), "") for s in SOURCES] +
            [("la2_api.cpp", tuple(extra) + ("-DLA2_TEST_HOOKS",), ".hooks"), ("la2_stream.hip", tuple(extra), "")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    if verbose:
        for _, msgs in results:
            if msgs.strip():
                print(msgs, file=sys.stderr)
    objs = [o for o, _ in results[:len(SOURCES)]]
    _link(objs, LIB)
    api = objs.index(os.path.join(OBJDIR, "la2_api.cpp.o"))
    # the test build: the API with the plan overrides, and the measurement stream
    _link(objs[:api] + [results[-2][0]] + objs[api + 1:] + [results[-1][0]], TEST_LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True, extra=sys.argv[1:]))
