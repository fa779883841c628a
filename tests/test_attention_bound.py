"""The attention parity bound is tight enough to matter (CPU only).

The GPU tests accept an output element when |gpu - ref| <= 2^-8 (sum_j p_j
|v_j,d| + |ref|) (tests/test_attention_gpu.py).  Here, at the full
64-sequence x 4096-key E4M3 workload, slips that a split-KV kernel could make
are planted in a copy of the oracle's source (one key lost at a key-range
edge, the last key lost, the scores scaled by 1.02), and the bound must
reject each of them on many elements.  The bound must also accept the oracle
itself evaluated a second way (float32 weights rounded to bf16, as the
kernel rounds them), which is the error it was derived for.
"""
from __future__ import annotations

import types

import numpy as np
import pytest

from mla_decode_concat_amd import inputs as I
from oracle import attention as A
from tests._util import bits
from tests.test_attention_gpu import tolerance

W = I.ATTN_WORKLOADS["attn_b64_l4096_h16_kvfp8"]

# (name, text in the oracle source, replacement): each a slip of the kind a
# split of the keys into ranges of 1024 could make
SLIPS = [
    ("key_at_range_edge_lost", "j = np.arange(L)",
     "j = np.delete(np.arange(L), 1024) if L > 1024 else np.arange(L)"),
    ("last_key_lost", "j = np.arange(L)", "j = np.arange(max(L - 1, 1))"),
    ("scores_scaled_2_percent", "s = (qd[b] @ rows.T) * sm_scale", "s = (qd[b] @ rows.T) * (sm_scale * 1.02)"),
]


@pytest.fixture(scope="module")
def full_workload():
    inp = I.make_attn_inputs(W)
    args = (bits(inp["q"]), bits(inp["cache"]), inp["block_table"].numpy(), inp["seq_lens"].numpy(),
            W.sm_scale)
    kw = dict(q_scale=None, kv_scale=W.kv_scale)
    ref, mag = A.mla_decode_attention(*args, **kw, with_abs=True)
    return args, kw, ref, tolerance(ref, mag)


def _mutant(old: str, new: str):
    text = open(A.__file__).read()
    assert text.count(old) == 1, old
    mod = types.ModuleType("attention_slip")
    exec(compile(text.replace(old, new), "attention_slip.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", SLIPS, ids=[s[0] for s in SLIPS])
def test_bound_rejects_slip_at_full_size(full_workload, name, old, new):
    args, kw, ref, tol = full_workload
    got = _mutant(old, new).mla_decode_attention(*args, **kw)
    n_bad = int((np.abs(got - ref) > tol).sum())
    print(f"{name}: {n_bad} of {ref.size} elements outside the bound")
    # "many": at least 2000 elements (0.4 % of the 524 288 outputs), and in
    # at least 10 of the 64 x 16 (sequence, head) pairs
    pairs = int((np.abs(got - ref) > tol).any(axis=2).sum())
    assert n_bad >= 2000 and pairs >= 10, (name, n_bad, pairs)


def test_bound_accepts_bf16_rounded_weights(full_workload):
    """The same attention with each unnormalised weight rounded to bf16 before
    the value product (the normaliser unrounded), then the output rounded to
    bf16: the error the bound was derived for, which it must accept."""
    import torch
    (q, cache, table, lens, sm_scale), kw, ref, tol = full_workload
    qd = A.bf16_decode(q)
    bs = cache.shape[1]
    got = np.zeros_like(ref)
    for b in range(q.shape[0]):
        L = int(lens[b])
        j = np.arange(L)
        rows = A.e4m3_decode(cache[table[b][j // bs], j % bs, :]) * kw["kv_scale"]
        s = (qd[b] @ rows.T) * sm_scale
        p = np.exp(s - s.max(axis=1, keepdims=True)).astype(np.float32)
        pb = torch.from_numpy(p).to(torch.bfloat16).double().numpy()
        got[b] = (pb @ rows[:, :512]) / p.astype(np.float64).sum(axis=1, keepdims=True)
    got = torch.from_numpy(got).to(torch.bfloat16).double().numpy()
    err = np.abs(got - ref)
    assert np.all(err <= tol), float((err / tol).max())
    # and it is not vacuous: the rounding uses a good part of the allowance
    assert float((err / tol).max()) > 0.2
