"""Host-side tests (no GPU) of the epilogue fused into the W_UK product:
its plan struct matches the header, validation returns the documented codes
without launching, and the plan covers every (head, token range, column
group) tile with the documented workgroup mapping."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import mla_decode_concat_amd as M
from mla_decode_concat_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_dq.h")

BASE = 1 << 36
GAP = 1 << 32


def test_uk_plan_struct_matches_header_layout():
    text = open(HEADER).read()
    body = re.search(r"typedef struct mla_dq_uk_launch_plan \{(.*?)\} mla_dq_uk_launch_plan;", text, re.S).group(1)
    fields = re.findall(r"(int32_t|int64_t)\s+(\w+);", body)
    want = [(n, ctypes.c_int32 if t == "int32_t" else ctypes.c_int64) for t, n in fields]
    assert [(n, t) for n, t in B.UkLaunchPlan._fields_] == want


def _dims(T=4, H=2, NB=1, BS=64, maxpos=16):
    """q_nope and q_pe as views of a [T, H, 192] q projection output."""
    d = B.Dims()
    d.num_tokens, d.num_heads, d.num_blocks, d.block_size, d.max_position = T, H, NB, BS, maxpos
    d.ql_nope_stride_t, d.ql_nope_stride_h = H * 192, 192
    d.q_pe_stride_t, d.q_pe_stride_h = H * 192, 192
    d.kv_c_stride_t, d.k_pe_stride_t = 512, 64
    return d


def _ptrs():
    names = ["q_out", "q_nope", "w_uk_t", "q_pe", "kv_c", "k_pe", "cache", "slots", "pos", "cs", "qs", "ks"]
    return {n: BASE + i * GAP for i, n in enumerate(names)}


def _call(p, flags, dims):
    return B.raw_uk_call(p["q_out"], p["q_nope"], p["w_uk_t"], p["q_pe"], p["kv_c"], p["k_pe"], p["cache"],
                         p["slots"], p["pos"], p["cs"], p["qs"], p["ks"], flags, dims, None) \
        if dims is not None else B.load().mla_decode_uk_q_concat_kv_insert(
            *(p[n] for n in ("q_out", "q_nope", "w_uk_t", "q_pe", "kv_c", "k_pe", "cache", "slots", "pos", "cs",
                             "qs", "ks")), ctypes.c_uint32(flags), None, None)


def test_null_dims():
    assert _call(_ptrs(), 0, None) == B.ERR_NULL


@pytest.mark.parametrize("flags", [M.Q_ROWS_ONLY, M.CACHE_ROWS_ONLY, M.FORCE_MID_T, 1 << 15,
                                   M.FORCE_SMALL_T | M.FORCE_LARGE_T, M.FORCE_STREAM | M.FORCE_CACHED,
                                   M.ROPE_GPTJ])
def test_bad_flags(flags):
    assert _call(_ptrs(), flags, _dims()) == B.ERR_FLAGS


@pytest.mark.parametrize("flags", [M.Q_ROWS_ONLY, M.CACHE_ROWS_ONLY, M.FORCE_MID_T])
def test_plan_rejects_subsets_and_mid_mapping(flags):
    with pytest.raises(M.MlaDqError) as e:
        M.uk_plan(_dims(), flags)
    assert e.value.code == B.ERR_FLAGS


def test_zero_tokens_is_a_no_op_even_with_null_pointers():
    p = {k: None for k in _ptrs()}
    assert _call(p, M.ROPE | M.Q_FP8 | M.KV_FP8, _dims(T=0)) == B.OK


@pytest.mark.parametrize("name", ["q_out", "q_nope", "w_uk_t", "q_pe", "kv_c", "k_pe", "cache", "slots"])
def test_null_required_pointer(name):
    p = _ptrs()
    p[name] = None
    assert _call(p, 0, _dims()) == B.ERR_NULL


@pytest.mark.parametrize("name,off", [("w_uk_t", 8), ("q_nope", 2), ("q_out", 8)])
def test_misaligned_pointer(name, off):
    p = _ptrs()
    p[name] += off
    assert _call(p, 0, _dims()) == B.ERR_ALIGN


def test_misaligned_q_nope_stride():
    d = _dims()
    d.ql_nope_stride_h += 4
    assert _call(_ptrs(), 0, d) == B.ERR_ALIGN


@pytest.mark.parametrize("out", ["q_out", "cache"])
def test_output_over_the_weights_is_rejected(out):
    """W_UK counts as an input: H * 512 * 128 bf16, the last 16 bytes included."""
    H = 3
    p = _ptrs()
    p[out] = p["w_uk_t"] + H * 512 * 128 * 2 - 16
    assert _call(p, 0, _dims(H=H)) == B.ERR_ALIAS
    p[out] = p["w_uk_t"] + H * 512 * 128 * 2           # just past it
    assert _call(p, 0, _dims(H=H)) != B.ERR_ALIAS


@pytest.mark.parametrize("out", ["q_out", "cache"])
def test_output_over_the_end_of_q_nope_is_rejected(out):
    """q_nope's extent ends 128 elements past its last row's start."""
    T, H = 4, 2
    p = _ptrs()
    last_row = ((T - 1) * H * 192 + (H - 1) * 192) * 2
    p[out] = p["q_nope"] + last_row + 256 - 16
    assert _call(p, 0, _dims(T=T, H=H)) == B.ERR_ALIAS
    p[out] = p["q_nope"] + last_row + 256
    assert _call(p, 0, _dims(T=T, H=H)) != B.ERR_ALIAS


def _algorithmic_bytes(T, H, flags):
    """Reads: q_nope (256 B per query row), q_pe (128 B), W_UK once
    (H * 128 KiB), kv_c + k_pe (1152 B per token), the slot (8 B) and, with
    the rotation, the position (8 B) and the table row (256 or 128 B).
    Writes: the 576-element rows of q and the cache."""
    table_row = 128 if flags & M.TABLE_BF16 else 256
    read = T * H * (256 + 128) + H * 512 * 128 * 2 + T * (1152 + 8) + (T * (8 + table_row) if flags & M.ROPE else 0)
    write = T * 576 * (H * (1 if flags & M.Q_FP8 else 2) + (1 if flags & M.KV_FP8 else 2))
    return read + write


@pytest.mark.parametrize("T,H", [(1, 16), (5, 3), (64, 16), (255, 16), (256, 16), (256, 128), (1000, 5),
                                 (8192, 16), (4096, 1), (16384, 128), (300, 64), (37, 100), (9, 128)])
@pytest.mark.parametrize("flags", [0, M.ROPE | M.KV_FP8, M.ROPE | M.Q_FP8, M.ROPE | M.TABLE_BF16 | M.Q_FP8 | M.KV_FP8])
def test_plan_counts_and_coverage(T, H, flags):
    p = M.uk_plan(_dims(T=T, H=H, NB=(T + 63) // 64 + 1, maxpos=32768), flags)
    assert p.block_threads == 256
    waves = p.block_threads // 64
    assert p.mapping == (1 if T * H >= p.large_rows_min else 0)
    if p.mapping:   # two 16-column blocks per wavefront from 64 tokens up to 16384 query rows
        assert p.n_blocks == (2 if T * H <= 16384 and T >= 64 else 4)
    else:   # one 16-column block per wavefront for at most 32 (head, 16-token range) units
        assert p.n_blocks == (1 if H * math.ceil(T / 16) <= 32 else 2)
    assert p.tail_steps == (2 if p.mapping else 1)
    assert p.column_groups * waves * 16 * p.n_blocks == 512
    # tokens per product workgroup: 16 for the latency configuration; for the
    # throughput one the largest of 128, 64, 32 that keeps >= 256 product
    # workgroups, else 16
    if p.mapping == 0:
        assert p.tokens_per_group == 16
    else:
        want = 16
        for tpg in (128, 64, 32):
            if H * math.ceil(T / tpg) * p.column_groups >= 256:
                want = tpg
                break
        assert p.tokens_per_group == want
    assert p.units == H * math.ceil(T / p.tokens_per_group)
    assert p.product_blocks % 8 == 0
    assert p.tail_blocks == math.ceil(T * (H + 1) / (p.block_threads // 8 * p.tail_steps))
    assert p.cache_blocks == math.ceil(T / waves)
    assert p.grid_blocks == p.product_blocks + p.tail_blocks + p.cache_blocks
    assert p.bytes == _algorithmic_bytes(T, H, flags)
    assert p.flops == 2 * T * H * 128 * 512
    assert p.streaming == (1 if p.bytes >= p.stream_bytes_min else 0)
    # the documented workgroup -> (head, token range, column group) mapping
    # reaches every triple exactly once; the other workgroups exit.  From 64
    # heads each XCD takes a contiguous block of head-major units, else unit
    # u = range * H + head goes to XCD u % 8.
    ranges = math.ceil(T / p.tokens_per_group)
    assert p.head_major == (1 if H >= 64 else 0)
    per_xcd = math.ceil(p.units / 8)
    seen = set()
    for g in range(p.product_blocks):
        xcd, m = g % 8, g // 8
        group = m % p.column_groups
        if p.head_major:
            pos = m // p.column_groups
            unit = xcd * per_xcd + pos
            if pos >= per_xcd or unit >= p.units:
                continue
            h, r = divmod(unit, ranges)
        else:
            unit = 8 * (m // p.column_groups) + xcd
            if unit >= p.units:
                continue
            r, h = divmod(unit, H)
        assert 0 <= h < H and 0 <= r < ranges
        assert (h, r, group) not in seen
        seen.add((h, r, group))
    assert len(seen) == p.units * p.column_groups == H * ranges * p.column_groups


def test_plan_overrides():
    d = _dims(T=64, H=16, maxpos=32768)
    assert M.uk_plan(d, 0).mapping == 0
    assert M.uk_plan(d, M.FORCE_LARGE_T).mapping == 1
    assert M.uk_plan(d, M.FORCE_STREAM).streaming == 1
    d = _dims(T=8192, H=16, NB=130, maxpos=32768)
    assert M.uk_plan(d, M.ROPE | M.KV_FP8).streaming == 1
    assert M.uk_plan(d, M.ROPE | M.KV_FP8 | M.FORCE_CACHED).streaming == 0
    assert M.uk_plan(d, M.FORCE_SMALL_T).mapping == 0


def test_plan_default_thresholds():
    """Without the environment overrides: the throughput configuration from
    1025 query rows, one 16-column block per wavefront in the latency one
    for at most 32 units, streaming from the epilogue's 80 MiB."""
    if any(v in os.environ for v in ("MLA_DQ_UK_LARGE_ROWS_MIN", "MLA_DQ_STREAM_BYTES_MIN")):
        pytest.skip("threshold overridden in the environment")
    for T, H, want in [(64, 16, 0), (65, 16, 1), (72, 16, 1), (8, 128, 0), (9, 128, 1), (1024, 1, 0), (1025, 1, 1)]:
        p = M.uk_plan(_dims(T=T, H=H, NB=(T + 63) // 64 + 1, maxpos=32768), M.ROPE | M.Q_FP8 | M.KV_FP8)
        assert p.large_rows_min == 1025 and p.mapping == want
    for T, H, nb in [(1024, 16, 2), (1025, 16, 4), (128, 128, 2), (129, 128, 4), (64, 128, 2), (63, 128, 4),
                     (65, 16, 2)]:
        p = M.uk_plan(_dims(T=T, H=H, NB=(T + 63) // 64 + 1, maxpos=32768), M.ROPE)
        assert p.mapping == 1 and p.n_blocks == nb and p.column_groups == 512 // (4 * 16 * nb)
    for T, H, nb in [(1, 16, 1), (32, 16, 1), (33, 16, 2), (64, 16, 2), (1, 32, 1), (1, 33, 2), (1, 128, 2)]:
        p = M.uk_plan(_dims(T=T, H=H, NB=(T + 63) // 64 + 1, maxpos=32768), M.ROPE)
        assert p.mapping == 0 and p.n_blocks == nb and p.column_groups == 512 // (4 * 16 * nb)
    p = M.uk_plan(_dims(T=2048, H=16, NB=33, maxpos=32768), M.ROPE)
    assert p.stream_bytes_min == 80 << 20 and p.streaming == 0
