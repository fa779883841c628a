"""The C ABI from a plain C11 program (no GPU): the public headers compile
with gcc -std=c11 -pedantic -Werror, the program links against the in-tree
libmla_dq.so, and calls that need no device work behave as declared: the
host-only launch plans, the error strings, and argument checks that return
before anything is launched."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import mla_decode_concat_amd as M
from mla_decode_concat_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mla_dq.h"
#include "mla_attn.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

int main(void) {
    mla_dq_dims d;
    memset(&d, 0, sizeof d);
    d.num_tokens = 8192; d.num_heads = 16; d.num_blocks = 4096; d.block_size = 64; d.max_position = 32768;
    d.ql_nope_stride_t = 16 * 512; d.ql_nope_stride_h = 512; d.q_pe_stride_t = 16 * 64; d.q_pe_stride_h = 64;
    d.kv_c_stride_t = 512; d.k_pe_stride_t = 64;
    mla_dq_launch_plan p;
    CHECK(mla_dq_plan(&d, MLA_DQ_ROPE | MLA_DQ_KV_FP8, &p) == MLA_DQ_OK);
    CHECK(p.bytes == 318373888LL);
    CHECK(p.grid_blocks > 0 && p.total_rows == 8192LL * 17);
    CHECK(p.streaming == 1 && p.stream_bytes_min == (80LL << 20));   /* default streaming threshold */
    CHECK(mla_dq_plan(&d, 1u << 30, &p) == MLA_DQ_ERR_FLAGS);
    CHECK(mla_dq_plan(NULL, 0, &p) == MLA_DQ_ERR_NULL);

    /* the fused call's plan: q_nope as views of a [T, H, 192] buffer */
    d.ql_nope_stride_t = 16 * 192; d.ql_nope_stride_h = 192; d.q_pe_stride_t = 16 * 192; d.q_pe_stride_h = 192;
    mla_dq_uk_launch_plan u;
    CHECK(mla_dq_uk_plan(&d, MLA_DQ_ROPE | MLA_DQ_KV_FP8, &u) == MLA_DQ_OK);
    CHECK(u.mapping == 1 && u.flops == 2LL * 8192 * 16 * 128 * 512);
    CHECK(mla_dq_uk_plan(&d, MLA_DQ_Q_ROWS_ONLY, &u) == MLA_DQ_ERR_FLAGS);

    /* argument checks return before any launch */
    CHECK(mla_decode_q_concat_kv_insert(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                        0, &d, NULL) == MLA_DQ_ERR_NULL);
    CHECK(mla_decode_uk_q_concat_kv_insert(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                           NULL, 0, &d, NULL) == MLA_DQ_ERR_NULL);
    d.num_tokens = 0;   /* nothing to do: success before any pointer is needed, nothing launched */
    CHECK(mla_decode_q_concat_kv_insert(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                        0, &d, NULL) == MLA_DQ_OK);

    CHECK(strcmp(mla_dq_strerror(MLA_DQ_OK), "success") == 0);
    CHECK(strlen(mla_dq_strerror(MLA_DQ_ERR_ALIAS)) > 0);
    CHECK(strlen(mla_dq_source_digest()) == 32);

    mla_attn_dims a;
    memset(&a, 0, sizeof a);
    a.batch = 64; a.num_heads = 16; a.num_blocks = 4096; a.block_size = 64; a.max_blocks_per_seq = 64;
    a.max_seq_len = 4096;
    mla_attn_plan ap;
    CHECK(mla_decode_attention_plan(&a, MLA_ATTN_KV_FP8, &ap) == MLA_DQ_OK);
    CHECK(ap.splits == 4 && ap.combine == 1 && ap.workgroups == 256 && ap.block_threads == 512);
    CHECK(mla_decode_attention_workspace_size(&a, MLA_ATTN_KV_FP8) == (size_t)ap.workspace_bytes);
    a.batch = 1; a.max_blocks_per_seq = 16; a.max_seq_len = 1024;   /* 16 ranges of 64 keys: no loaders */
    CHECK(mla_decode_attention_plan(&a, MLA_ATTN_KV_FP8, &ap) == MLA_DQ_OK);
    CHECK(ap.splits == 16 && ap.keys_per_split == 64 && ap.block_threads == 256);
    printf("%s\n", fails ? "failed" : "ok");
    return fails != 0;
}
"""


def test_c_program_against_the_library(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    M.load()                                   # the in-tree library exists and matches the sources
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(B.LIB)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-lmla_dq", "-Wl,-rpath," + libdir,
           "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    for var in ("MLA_DQ_STREAM_BYTES_MIN", "MLA_ATTN_TARGET_WGS", "MLA_DQ_UK_LARGE_ROWS_MIN",
                "MLA_DQ_SMALL_ROWS_MAX", "MLA_DQ_MID_ROWS_MAX"):
        env.pop(var, None)                     # the checks above expect the library's defaults
    env["LD_LIBRARY_PATH"] = ":".join(p for p in ("/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")) if p)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
