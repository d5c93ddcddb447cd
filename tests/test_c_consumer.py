"""The boundary is plain C: a C99 program that includes include/la2.h (with -Wall -Wextra -Werror)
links against the built library and calls it without any C++ or Python in between.  Only calls
that need no GPU are made: the version, the status strings, workspace sizes and argument checks
that fail before anything is enqueued."""
import os
import shutil
import subprocess

import pytest

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "la2.h"

int main(void) {
    char buf[64];
    int bad = 0;
    printf("abi %d\n", la2_abi_version());
    if (strlen(la2_status_string(LA2_OK)) == 0) bad = 1;
    /* no q: rejected before any device work */
    int st = la2_forward(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 64, 64, 64, LA2_BF16, NULL, 0, NULL);
    printf("null %d\n", st);
    /* unsupported head size */
    st = la2_forward((void *)0x100000, (void *)0x200000, (void *)0x300000, NULL, (void *)0x400000,
                     1, 1, 64, 96, 64, 64, LA2_BF16, NULL, 0, NULL);
    printf("unsupported %d\n", st);
    size_t w = la2_workspace_bytes(1, 16, 131072, 128, 128, 128, LA2_BF16, 1);
    printf("workspace %zu\n", w);
    snprintf(buf, sizeof buf, "%s", la2_status_string(LA2_ERR_ALIAS));
    printf("alias %s\n", buf);
    return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_plain_c_program_uses_the_library(tmp_path):
    la2.load_library()
    src = tmp_path / "use_la2.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_la2"
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}", str(src),
           f"-L{libdir}", "-lla2", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert int(got["abi"]) == binding.LA2_ABI_VERSION
    assert int(got["null"]) == 1           # LA2_ERR_NULL_POINTER
    assert int(got["unsupported"]) == 3    # LA2_ERR_UNSUPPORTED
    assert int(got["workspace"]) == la2.la2_workspace_bytes(1, 16, 131072, 128, 128, 128, binding.LA2_BF16, True) > 0
    assert got["alias"] == la2.la2_status_string(5)
