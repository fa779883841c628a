"""CPU oracle for MLA decode attention over the paged latent cache -- TEST
INFRASTRUCTURE ONLY (only tests/, smoke() and bench.py's CPU baseline use it).

The consumer of the epilogue (prhub summary of vLLM PR #54896, "implementation
breakdown" item 2: the epilogue's output feeds the downstream FMHA of the
decode step).  With the weight absorption of multi-head latent attention,
every head's query is a 576-wide latent row and every cached token is one
576-wide latent row shared by all heads: the key is the whole row, the value
its first 512 elements.  For sequence b with L = seq_lens[b] cached tokens and
head h:

    row_j   = cache[block_table[b, j // bs], j % bs, :]          j < L
    s_j     = sm_scale * <q[b, h, :], row_j>                    (576 terms)
    out[b, h, :] = sum_j softmax(s)_j * row_j[0:512]            (zeros if L == 0)

E4M3 operands are decoded from their codes (OCP OFP8 E4M3) and multiplied by
their per-tensor scale.  Everything is evaluated in float64.

Parity status: pinned in tests/test_attention_oracle.py (single key, repeated
keys, zero query, two-key closed form, page-order invariance, score-shift
invariance, torch scaled_dot_product_attention, every E4M3 code).
"""
from __future__ import annotations

import numpy as np

NOPE = 512
ROW = 576


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (bf16 is the top half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 from the OCP definition: sign, 4-bit exponent
    (bias 7), 3-bit mantissa; exponent 0 is subnormal (m * 2^-9);
    S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, v)


def mla_decode_attention(q: np.ndarray, cache: np.ndarray, block_table: np.ndarray,
                         seq_lens: np.ndarray, sm_scale: float, q_scale: float | None = None,
                         kv_scale: float | None = None, with_abs: bool = False):
    """Reference attention in float64.

    q            [B, H, 576] bf16 bit patterns (uint16) or E4M3 codes (uint8)
    cache        [num_blocks, bs, 576] bf16 bit patterns (uint16) or E4M3 codes (uint8)
    block_table  [B, max_blocks] int, seq_lens [B] int
    q_scale / kv_scale: per-tensor scales of E4M3 operands
    Returns out [B, H, 512] float64; with ``with_abs`` also the same weighted
    sum over the absolute values, sum_j softmax(s)_j * |row_j[0:512]|, which
    scales the rounding error of any evaluation of the weighted sum.
    """
    def decode(x, scale):
        if x.dtype == np.uint8:
            return e4m3_decode(x) * float(scale)
        return bf16_decode(x)

    B, H = q.shape[0], q.shape[1]
    bs = cache.shape[1]
    qd = decode(q, q_scale)
    out = np.zeros((B, H, NOPE), dtype=np.float64)
    mag = np.zeros((B, H, NOPE), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        j = np.arange(L)
        pages = np.asarray(block_table[b])[j // bs]
        rows = decode(cache[pages, j % bs, :], kv_scale)            # [L, 576]
        s = (qd[b] @ rows.T) * sm_scale                               # [H, L]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[b] = p @ rows[:, :NOPE]
        if with_abs:
            mag[b] = p @ np.abs(rows[:, :NOPE])
    return (out, mag) if with_abs else out
