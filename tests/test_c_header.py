"""include/attn.h is a C header, not only a C++ one: a C99 program that includes it
compiles with warnings as errors, links against libattn.so, and sees the documented host
behaviour (a refused argument before any HIP call, the thread's error text, the workspace
size).  CPU only: nothing here reaches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "transformer_attention_03_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "attn.h"

int main(void) {
    /* head_dim 96 is not built: refused before any HIP call */
    int rc = attn_decode((const float *)0x10000, (const void *)0x10000, (const void *)0x10000,
                         (float *)0x10000, 32, 8, 96, 4096, 0, 0.0f, 0.125f,
                         (void *)0x10000, (size_t)1 << 20, NULL);
    const char *msg = attn_last_error();
    size_t ws = attn_decode_workspace_bytes(1, 32, 8, 128, 4096);
    attn_dtype dt = ATTN_F16;
    printf("rc=%d unsupported=%d ws_nonzero=%d dtype=%d msg_has_head_dim=%d\n", rc,
           rc == ATTN_ERR_UNSUPPORTED, ws > 0, (int)dt, strstr(msg, "head_dim") != NULL);
    return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    lib = os.path.join(PKG, "libattn.so")
    if not os.path.exists(lib):
        pytest.skip("libattn.so not built")
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", PKG, "-lattn", "-Wl,-rpath," + PKG], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "unsupported=1 ws_nonzero=1 dtype=1 msg_has_head_dim=1" in out.stdout, out.stdout
