"""include/msa.h as a C interface, on the CPU: it compiles as strict C99 and as C++, a C program links
against libmsa.so and gets the documented status codes back, and the struct layouts the C
compiler gives match the ones the Python binding declares."""
import ctypes
import os
import shutil
import subprocess

import pytest

from block_sparse_long_msa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(_lib.LIB_PATH)

C_PROGRAM = r"""
#include <stddef.h>
#include <stdio.h>
#include "msa.h"

int main(void) {
  printf("batch %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(msa_batch), offsetof(msa_batch, num_requests),
         offsetof(msa_batch, num_queries), offsetof(msa_batch, max_blocks), offsetof(msa_batch, max_q_per_request),
         offsetof(msa_batch, block_table), offsetof(msa_batch, ctx_len), offsetof(msa_batch, cu_q),
         offsetof(msa_batch, q_pos));
  printf("cache %zu %zu %zu %zu %zu %zu %zu\n", sizeof(msa_cache), offsetof(msa_cache, data),
         offsetof(msa_cache, num_pages), offsetof(msa_cache, block_size), offsetof(msa_cache, num_heads),
         offsetof(msa_cache, head_dim), offsetof(msa_cache, page_stride));
  printf("version %d\n", msa_version());
  printf("status %s\n", msa_status_string(MSA_ERR_WORKSPACE_TOO_SMALL));
  /* rejected on the host before any launch: no device is touched */
  msa_status s = msa_lse_merge(-1, 4, 8, 128, NULL, NULL, NULL, NULL, NULL);
  printf("merge %d %s\n", (int)s, msa_last_error());
  s = msa_topk_blocks(NULL, 8, NULL, 16, NULL, NULL, NULL);
  printf("topk %d\n", (int)s);
  return 0;
}
"""


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_header_compiles_as_strict_c_and_cpp(tmp_path):
    _need("gcc")
    _need("g++")
    src = tmp_path / "h.c"
    src.write_text('#include "msa.h"\nint main(void) { return 0; }\n')
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", INCLUDE, str(src)],
                ["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c++", "-I",
                 INCLUDE, str(src)]):
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr


def test_c_program_links_and_layouts_match_the_binding(tmp_path):
    _need("gcc")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmsa.so is not built: run `python -m block_sparse_long_msa_amd.build`")
    src, exe = tmp_path / "p.c", tmp_path / "p"
    src.write_text(C_PROGRAM)
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", INCLUDE, str(src), "-o", str(exe), "-L", LIBDIR,
                          "-lmsa", f"-Wl,-rpath,{LIBDIR}"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    out = dict(line.split(" ", 1) for line in run.stdout.strip().splitlines())

    B, C = _lib.MsaBatch, _lib.MsaCache
    want_b = [ctypes.sizeof(B)] + [getattr(B, f).offset for f, _ in B._fields_]
    want_c = [ctypes.sizeof(C)] + [getattr(C, f).offset for f, _ in C._fields_]
    assert [int(v) for v in out["batch"].split()] == want_b
    assert [int(v) for v in out["cache"].split()] == want_c
    assert int(out["version"]) == _lib.load().msa_version()
    assert out["status"] == "MSA_ERR_WORKSPACE_TOO_SMALL"
    assert out["merge"].startswith("1 ") and "rows" in out["merge"]
    assert out["topk"] == "1"
