"""include/s3r.h is a C header and libs3r.so a C library: a C99 program (gcc,
-pedantic -Werror) and a C++ program include the header, link the library
directly (no Python, no torch) and call it. No GPU: the calls are host queries
(version, status text, workspace sizes) and argument checks that fail before any
launch. The workspace sizes the C program prints must equal the ones the Python
binding reports for the same shapes."""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "s3r.h"

int main(void) {
  s3r_paged_kv kv;
  int ok = 1;
  size_t ws_verify, ws_accept;
  memset(&kv, 0, sizeof kv);
  printf("version %d\n", (int)s3r_version());
  printf("status %s|%s|%s|%s|%s\n", s3r_status_string(S3R_SUCCESS), s3r_status_string(S3R_ERROR_INVALID_VALUE),
         s3r_status_string(S3R_ERROR_NOT_SUPPORTED), s3r_status_string(S3R_ERROR_INSUFFICIENT_WORKSPACE),
         s3r_status_string(S3R_ERROR_HIP));
  /* host-side checks: NULL buffers are rejected before any launch */
  if (s3r_select_budget(NULL, NULL, 4, 100, 16, 0.05, NULL, NULL, 8, NULL, 0, NULL) != S3R_ERROR_INVALID_VALUE) ok = 0;
  if (s3r_dense_verify_attn(&kv, 4, 16, 5, NULL, 0.125f, NULL, NULL, NULL, 0, NULL) != S3R_ERROR_INVALID_VALUE) ok = 0;
  if (s3r_spec_accept(4, 4, 1000, S3R_BF16, NULL, NULL, NULL, NULL, NULL, 1.0f, NULL, NULL, NULL, NULL, 0, NULL) !=
      S3R_ERROR_INVALID_VALUE)
    ok = 0;
  /* a cache descriptor of a 16K-token layer (its pointers are never dereferenced on the host) */
  kv.k_cache = (void*)(size_t)0x10000;
  kv.v_cache = (void*)(size_t)0x20000;
  kv.page_table = (const int32_t*)(size_t)0x30000;
  kv.ctx_lens = (const int32_t*)(size_t)0x40000;
  kv.num_blocks = 66115;
  kv.num_kv_heads = 8;
  kv.page_size = 16;
  kv.head_dim = 128;
  kv.max_pages_per_seq = 1033;
  kv.dtype = S3R_BF16;
  kv.page_size = 32;
  if (s3r_dense_verify_attn(&kv, 64, 16, 5, (const void*)(size_t)0x50000, 0.125f, (void*)(size_t)0x60000, NULL, NULL,
                            0, NULL) != S3R_ERROR_NOT_SUPPORTED)
    ok = 0;
  kv.page_size = 16;
  ws_verify = s3r_dense_verify_workspace_size(&kv, 64, 32, 7);
  ws_accept = s3r_spec_accept_workspace_size(64, 4, 151936);
  printf("ws_verify %zu\nws_accept %zu\n", ws_verify, ws_accept);
  if (ws_accept == 0) ok = 0;
  printf("%s\n", ok ? "C_CONSUMER_OK" : "C_CONSUMER_FAIL");
  return ok ? 0 : 1;
}
"""

CXX_SOURCE = r"""
#include <cstdio>
#include "s3r.h"
int main() {
  std::printf("%s %d\n", s3r_status_string(S3R_ERROR_HIP), static_cast<int>(s3r_version()));
  return s3r_spec_accept_workspace_size(64, 4, 151936) > 0 ? 0 : 1;
}
"""


@pytest.fixture(scope="module")
def lib_path():
    from rl_rollout_amd import s3r
    return s3r.LIB_PATH


def _build_and_run(tmp_path, compiler, flags, source, name, lib):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    src = tmp_path / name
    src.write_text(source)
    exe = tmp_path / (name + ".out")
    libdir = os.path.dirname(lib)
    cmd = [compiler, *flags, "-I", INCLUDE, str(src), "-o", str(exe), "-L", libdir, "-l:" + os.path.basename(lib),
           "-Wl,-rpath," + libdir, "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_c99_program_links_and_calls_the_library(tmp_path, lib_path):
    from rl_rollout_amd import s3r
    out = _build_and_run(tmp_path, "gcc", ["-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror"], C_SOURCE,
                         "consumer.c", lib_path)
    lines = dict(l.split(" ", 1) for l in out.strip().splitlines() if " " in l)
    assert out.strip().splitlines()[-1] == "C_CONSUMER_OK", out
    assert int(lines["version"]) == s3r.raw["s3r_version"]()
    assert lines["status"] == "success|invalid value|not supported|insufficient workspace|HIP runtime error"
    # the same shapes through the Python binding (8B-like block of 7 rows over 32 q heads)
    kv = s3r.PagedKV(k_cache=0x10000, v_cache=0x20000, page_table=0x30000, ctx_lens=0x40000, num_blocks=66115,
                     num_kv_heads=8, page_size=16, head_dim=128, max_pages_per_seq=1033, dtype=1)
    assert int(lines["ws_verify"]) > 0  # two column tiles stage page log-sum-exps in the workspace
    assert int(lines["ws_verify"]) == s3r.raw["s3r_dense_verify_workspace_size"](ctypes.byref(kv), 64, 32, 7)
    assert int(lines["ws_accept"]) == s3r.spec_accept_workspace_size(64, 4, 151936)


def test_cxx_program_links_and_calls_the_library(tmp_path, lib_path):
    out = _build_and_run(tmp_path, "g++", ["-std=c++11", "-Wall", "-Wextra", "-Werror"], CXX_SOURCE, "consumer.cpp",
                         lib_path)
    assert out.startswith("HIP runtime error "), out
