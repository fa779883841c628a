"""Host-side tests of the decode-attention C ABI (include/mla_attn.h), no
GPU: flag and code values, the key-split plan, workspace sizing, and the
argument checks that return before anything is launched."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import mla_decode_concat_amd as M
from mla_decode_concat_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_attn.h")


def test_flag_and_code_values_match_header():
    text = open(HEADER).read()
    assert re.search(r"#define MLA_ATTN_Q_FP8\s+\(1u << 0\)", text) and M.ATTN_Q_FP8 == 1
    assert re.search(r"#define MLA_ATTN_KV_FP8\s+\(1u << 1\)", text) and M.ATTN_KV_FP8 == 2
    assert int(re.search(r"#define MLA_ATTN_ERR_WORKSPACE\s+(-?\d+)", text).group(1)) == \
        B.ERR_WORKSPACE
    assert int(re.search(r"#define MLA_ATTN_ERR_SCRATCH\s+(-?\d+)", text).group(1)) == B.ERR_SCRATCH
    assert re.search(r"#define MLA_ATTN_SCRATCH_BYTES\s+\(16u << 20\)", text) and B.SCRATCH_BYTES == 16 << 20


def test_default_plans_fit_the_scratch_buffer():
    """Every split the default plan makes fits the allocation-free entry
    point's buffer: at most 510 workgroups of 16 heads need records, the
    largest being 255 (sequence, head tile) pairs split in two."""
    worst = 0
    for B_ in list(range(1, 300)) + [511, 1024]:
        for H in (1, 15, 16, 17, 31, 32, 48, 64, 128):
            for L in (64, 65, 1000, 4096, 1 << 16, 1 << 20):
                MB = (L + 63) // 64
                ws = M.attn_workspace_size(dims(B_, H, NB=MB, MB=MB, L=L), M.ATTN_KV_FP8)
                worst = max(worst, ws)
    assert 0 < worst <= B.SCRATCH_BYTES
    assert worst == 255 * 16 * 2 * (512 + 2) * 4


def test_noalloc_refuses_a_split_beyond_the_scratch_in_fresh_process():
    """With the workgroup target raised the split can need more than the
    buffer: the call returns MLA_ATTN_ERR_SCRATCH before touching the GPU."""
    code = ("import ctypes, mla_decode_concat_amd as M; from mla_decode_concat_amd import _binding as B;"
            "d=M.AttnDims(); d.batch=64; d.num_heads=128; d.num_blocks=4096; d.block_size=64;"
            "d.max_blocks_per_seq=64; d.max_seq_len=4096; lib=B._attn_lib();"
            "p=[(1<<36)+i*(1<<32) for i in range(7)];"
            "print(M.attn_plan(d,2).workspace_bytes, lib.mla_decode_attention_noalloc(*p, ctypes.c_float(0.07),"
            " ctypes.c_uint32(2), ctypes.byref(d), None))")
    env = dict(os.environ, MLA_ATTN_TARGET_WGS="8192", PYTHONPATH=ROOT)
    out = subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True, check=True)
    need, rc = out.stdout.split()
    assert int(need) > B.SCRATCH_BYTES and int(rc) == B.ERR_SCRATCH


def test_plan_struct_matches_header_layout():
    text = open(HEADER).read()
    body = re.search(r"typedef struct mla_attn_plan \{(.*?)\} mla_attn_plan;", text, re.S).group(1)
    fields = re.findall(r"(int32_t|int64_t)\s+(\w+);", body)
    want = [(n, ctypes.c_int32 if t == "int32_t" else ctypes.c_int64) for t, n in fields]
    assert [(n, t) for n, t in B.AttnPlan._fields_] == want
    body = re.search(r"typedef struct mla_attn_dims \{(.*?)\} mla_attn_dims;", text, re.S).group(1)
    assert [n for n, _ in B.AttnDims._fields_] == re.findall(r"int64_t\s+(\w+);", body)


def dims(B_=4, H=16, NB=64, BS=64, MB=16, L=None):
    d = M.AttnDims()
    d.batch, d.num_heads, d.num_blocks, d.block_size = B_, H, NB, BS
    d.max_blocks_per_seq = MB
    d.max_seq_len = MB * BS if L is None else L
    return d


@pytest.mark.parametrize("B_,H,L", [(1, 16, 1), (1, 16, 64), (1, 16, 65), (1, 16, 1024),
                                    (64, 16, 4096), (64, 128, 4096), (13, 20, 4096),
                                    (512, 16, 300), (32, 256, 311), (3, 1, 0), (0, 16, 100)])
def test_plan_covers_every_key_once(B_, H, L):
    MB = max(1, (L + 63) // 64)
    for flags in (0, M.ATTN_KV_FP8, M.ATTN_Q_FP8 | M.ATTN_KV_FP8):
        p = M.attn_plan(dims(B_, H, MB=MB, L=L), flags)
        assert p.keys_per_split % 64 == 0 and p.keys_per_split >= 64
        assert p.splits >= 1
        # the ranges cover [0, L) and none starts past it (no idle split)
        assert p.splits * p.keys_per_split >= L
        assert L == 0 and p.splits == 1 or (p.splits - 1) * p.keys_per_split < L
        assert p.head_tiles == (H + 15) // 16
        assert p.workgroups == B_ * p.head_tiles * p.splits
        assert p.combine == (1 if p.splits > 1 else 0)
        ws = B_ * H * p.splits * (512 + 2) * 4 if p.combine else 0
        assert p.workspace_bytes == ws
        assert M.attn_workspace_size(dims(B_, H, MB=MB, L=L), flags) == ws
        # E4M3 cache: four compute plus four loader wavefronts, or four that
        # load their own tile when each range is one tile per wavefront;
        # bf16: four
        loaders = bool(flags & M.ATTN_KV_FP8) and p.keys_per_split > 64
        assert p.block_threads == (512 if loaders else 256) and p.target_workgroups == 256
        assert p.xcd_remap == (1 if p.head_tiles > 1 and p.workgroups % 8 == 0 else 0)


def test_plan_aims_at_the_target_workgroup_count():
    p = M.attn_plan(dims(64, 16, MB=64, L=4096), M.ATTN_KV_FP8)
    assert (p.splits, p.keys_per_split, p.workgroups) == (4, 1024, 256)
    p = M.attn_plan(dims(1, 16, MB=16, L=1024), M.ATTN_KV_FP8)
    assert (p.splits, p.keys_per_split) == (16, 64)      # at least 64 keys per range


def test_target_env_override_in_fresh_process():
    code = ("import mla_decode_concat_amd as M; d=M.AttnDims(); d.batch=64; d.num_heads=16;"
            "d.num_blocks=4096; d.block_size=64; d.max_blocks_per_seq=64; d.max_seq_len=4096;"
            "p=M.attn_plan(d,0); print(p.target_workgroups, p.splits, p.keys_per_split)")
    env = dict(os.environ, MLA_ATTN_TARGET_WGS="128", PYTHONPATH=ROOT)
    out = subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True, check=True)
    assert out.stdout.split() == ["128", "2", "2048"]


BASE = 1 << 36
GAP = 1 << 32


def _ptrs():
    names = ["out", "q", "cache", "bt", "lens", "qs", "ks", "ws"]
    return {n: BASE + i * GAP for i, n in enumerate(names)}


def _call(p, flags, d, ws_bytes=1 << 30, sm=0.07):
    lib = B._attn_lib()
    return lib.mla_decode_attention(p["out"], p["q"], p["cache"], p["bt"], p["lens"], p["qs"],
                                    p["ks"], ctypes.c_float(sm), p["ws"], ctypes.c_size_t(ws_bytes),
                                    ctypes.c_uint32(flags),
                                    ctypes.byref(d) if d is not None else None, None)


def test_null_dims_and_plan():
    assert _call(_ptrs(), 0, None) == B.ERR_NULL
    lib = B._attn_lib()
    assert lib.mla_decode_attention_plan(ctypes.byref(dims()), 0, None) == B.ERR_NULL
    assert lib.mla_decode_attention_workspace_size(None, 0) == 0


@pytest.mark.parametrize("flags", [1 << 2, 1 << 8, 1 << 31])
def test_bad_flags(flags):
    assert _call(_ptrs(), flags, dims()) == B.ERR_FLAGS


@pytest.mark.parametrize("field,value", [("batch", -1), ("num_heads", 0), ("num_blocks", 0),
                                         ("block_size", 0), ("max_blocks_per_seq", 0),
                                         ("max_seq_len", -1), ("max_seq_len", 16 * 64 + 1)])
def test_bad_dims(field, value):
    d = dims()
    setattr(d, field, value)
    assert _call(_ptrs(), 0, d) == B.ERR_DIM
    assert M.attn_workspace_size(d, 0) == 0


def test_zero_batch_is_a_no_op_even_with_null_pointers():
    p = {k: None for k in _ptrs()}
    assert _call(p, M.ATTN_Q_FP8 | M.ATTN_KV_FP8, dims(B_=0), ws_bytes=0) == B.OK


@pytest.mark.parametrize("name", ["out", "q", "cache", "bt", "lens", "ws"])
def test_null_required_pointer(name):
    p = _ptrs()
    p[name] = None
    assert _call(p, 0, dims()) == B.ERR_NULL


@pytest.mark.parametrize("flags,name", [(M.ATTN_Q_FP8, "qs"), (M.ATTN_KV_FP8, "ks")])
def test_null_scale_needed_by_flag(flags, name):
    p = _ptrs()
    p[name] = None
    assert _call(p, flags, dims()) == B.ERR_NULL


def test_workspace_too_small():
    d = dims()
    need = M.attn_workspace_size(d, 0)
    assert need > 0
    assert _call(_ptrs(), 0, d, ws_bytes=need - 1) == B.ERR_WORKSPACE


def test_workspace_may_be_null_when_none_is_needed():
    d = dims(B_=600, L=64, MB=1)          # one key range per sequence
    assert M.attn_workspace_size(d, 0) == 0
    p = _ptrs()
    p["ws"] = None
    p["out"] += 8                         # stop at the alignment check, before any launch
    assert _call(p, 0, d, ws_bytes=0) == B.ERR_ALIGN


@pytest.mark.parametrize("name,off", [("out", 8), ("q", 8), ("cache", 4), ("bt", 2), ("lens", 2),
                                      ("ws", 4)])
def test_misaligned_pointer(name, off):
    p = _ptrs()
    p[name] += off
    assert _call(p, 0, dims()) == B.ERR_ALIGN


@pytest.mark.parametrize("sm", [float("nan"), float("inf"), -float("inf")])
def test_bad_softmax_scale(sm):
    assert _call(_ptrs(), 0, dims(), sm=sm) == B.ERR_DIM


@pytest.mark.parametrize("moved,onto,off", [("out", "q", 16), ("q", "out", 4096), ("out", "cache", 0),
                                            ("out", "bt", 32), ("out", "lens", 0), ("ws", "out", 16),
                                            ("ws", "cache", 1 << 20), ("cache", "ws", 4096),
                                            ("bt", "ws", 64), ("out", "ks", 0)])
def test_output_or_workspace_overlapping_a_buffer(moved, onto, off):
    """out and the workspace are written while other workgroups read the
    inputs: any overlap with another buffer is refused before a launch."""
    p = _ptrs()
    p[moved] = p[onto] + off
    assert _call(p, M.ATTN_KV_FP8, dims()) == B.ERR_ALIAS



# ---- Python binding: argument checks that run before anything is launched ----

def _cpu_args(B_=2, H=16, NB=4, BS=64, MB=2, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16):
    return dict(out=torch.empty(B_, H, 512, dtype=torch.bfloat16),
                q=torch.zeros(B_, H, 576, dtype=q_dtype),
                cache=torch.zeros(NB, BS, 576, dtype=kv_dtype),
                block_table=torch.zeros(B_, MB, dtype=torch.int32),
                seq_lens=torch.ones(B_, dtype=torch.int32),
                q_scale=None, kv_scale=None)


def _validate(a):
    B._attn_validate(a["out"], a["q"], a["cache"], a["block_table"], a["seq_lens"],
                     a["q_scale"], a["kv_scale"])



@pytest.mark.parametrize("field,value,msg", [
    ("q", torch.zeros(2, 16, 512, dtype=torch.bfloat16), "q must be"),
    ("q", torch.zeros(2, 16, 576, dtype=torch.float16), "q must be bf16 or e4m3"),
    ("out", torch.empty(2, 16, 512, dtype=torch.float32), "out must be"),
    ("out", torch.empty(2, 8, 512, dtype=torch.bfloat16), "out must be"),
    ("cache", torch.zeros(4, 64, 512, dtype=torch.bfloat16), "cache must be"),
    ("cache", torch.zeros(4, 64, 576, dtype=torch.float32), "cache must be bf16 or e4m3"),
    ("block_table", torch.zeros(2, 2, dtype=torch.int64), "block_table must be"),
    ("block_table", torch.zeros(3, 2, dtype=torch.int32), "block_table must be"),
    ("seq_lens", torch.ones(2, dtype=torch.int64), "seq_lens must be"),
    ("seq_lens", torch.ones(3, dtype=torch.int32), "seq_lens must be"),
])
def test_binding_rejects_bad_arguments(field, value, msg):
    a = _cpu_args()
    a[field] = value
    with pytest.raises(ValueError, match=msg):
        _validate(a)


def test_binding_rejects_views_and_missing_scales():
    a = _cpu_args()
    a["q"] = torch.zeros(2, 576, 16, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        _validate(a)
    a = _cpu_args(kv_dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="kv_scale"):
        _validate(a)
    a = _cpu_args(q_dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="q_scale"):
        _validate(a)


def test_binding_requires_gpu_tensors():
    a = _cpu_args(q_dtype=torch.float8_e4m3fn, kv_dtype=torch.float8_e4m3fn)
    a["q_scale"] = torch.ones(1)
    a["kv_scale"] = torch.ones(1)
    with pytest.raises(ValueError, match="GPU"):
        _validate(a)
