"""The allocation-free decode attention entry point (include/mla_attn.h,
mla_decode_attention_noalloc), called through the C ABI: two calls in a row,
the second with a smaller input, each bit-identical to the workspace entry
point on the same inputs and within the attention bound of the oracle; the
shared scratch buffer keeps the first call's partial results, which must
not leak into the second."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_decode_concat_amd as M
from mla_decode_concat_amd import inputs as I
from tests.test_attention_gpu import DEV, announce, assert_close, oracle_out, to_device

pytestmark = pytest.mark.gpu


def _both_entry_points(w: I.AttnWorkload, seed: int):
    inp = I.make_attn_inputs(w, seed)
    d = to_device(inp)
    plan = M.attn_plan(M.AttnDims(w.batch, w.heads, w.num_blocks, w.block_size, w.max_blocks,
                                  w.max_blocks * w.block_size),
                       (M.ATTN_Q_FP8 if w.q_fp8 else 0) | (M.ATTN_KV_FP8 if w.kv_fp8 else 0))
    announce(f"no-alloc {w.describe()} splits={plan.splits} workspace={plan.workspace_bytes}")
    ref_out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device=DEV)
    ref_out.view(torch.int16).fill_(-1)
    M.mla_decode_attention(d["q"], d["cache"], d["block_table"], d["seq_lens"], w.sm_scale,
                           d["q_scale"], d["kv_scale"], out=ref_out)
    out = torch.empty_like(ref_out)
    out.view(torch.int16).fill_(-1)                        # NaN: every element must be written
    M.mla_decode_attention_noalloc(out, d["q"], d["cache"], d["block_table"], d["seq_lens"],
                                   w.sm_scale, d["q_scale"], d["kv_scale"])
    torch.cuda.synchronize()
    return inp, plan, out, ref_out


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 12 sequences up to 4096 keys, 16 ranges each (scratch in use)
    w1 = I.attn_custom(12, 16, (4096, 3000, 1, 0, 65, 2048, 4000, 17, 1024, 777, 4096, 129),
                       kv_fp8=True, name="noalloc1")
    inp1, plan1, out1, ref1 = _both_entry_points(w1, seed=41)
    assert plan1.workspace_bytes > 0
    assert torch.equal(out1.view(torch.int16), ref1.view(torch.int16))
    want1, tol1 = oracle_out(w1, inp1)
    assert_close(out1.float().cpu().numpy().astype(np.float64), want1, tol1, "no-alloc call 1")
    # second call, smaller: 3 sequences, 20 heads, E4M3 queries, fewer ranges
    # than the first call wrote
    w2 = I.attn_custom(3, 20, (700, 10, 1500), q_fp8=True, kv_fp8=True, name="noalloc2")
    inp2, plan2, out2, ref2 = _both_entry_points(w2, seed=42)
    assert 0 < plan2.workspace_bytes < plan1.workspace_bytes
    assert torch.equal(out2.view(torch.int16), ref2.view(torch.int16))
    want2, tol2 = oracle_out(w2, inp2)
    assert_close(out2.float().cpu().numpy().astype(np.float64), want2, tol2, "no-alloc call 2")


def test_noalloc_without_split_and_bf16_cache():
    """A batch large enough that every sequence is one range (no scratch
    needed), then a bf16 cache split into ranges."""
    w = I.attn_custom(300, 16, tuple(range(1, 601, 2)), kv_fp8=True, name="noalloc-direct")
    inp, plan, out, ref = _both_entry_points(w, seed=43)
    assert plan.workspace_bytes == 0
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    w = I.attn_custom(2, 16, (2000, 333), name="noalloc-bf16")
    inp, plan, out, ref = _both_entry_points(w, seed=44)
    assert plan.workspace_bytes > 0
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    want, tol = oracle_out(w, inp)
    assert_close(out.float().cpu().numpy().astype(np.float64), want, tol, "no-alloc bf16")
