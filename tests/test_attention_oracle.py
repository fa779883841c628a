"""Pins of the attention oracle (oracle/attention.py) against closed forms,
invariances and torch's scaled_dot_product_attention."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention as A
from mla_decode_concat_amd import inputs as I
from tests._util import bits


def _run(w, inp):
    return A.mla_decode_attention(bits(inp["q"]), bits(inp["cache"]), inp["block_table"].numpy(),
                                  inp["seq_lens"].numpy(), w.sm_scale,
                                  w.q_scale if w.q_fp8 else None, w.kv_scale if w.kv_fp8 else None)


def _rows(w, inp, b, fp8=None):
    bt, L = inp["block_table"][b].numpy(), int(inp["seq_lens"][b])
    j = np.arange(L)
    raw = bits(inp["cache"])[bt[j // w.block_size], j % w.block_size]
    if raw.dtype == np.uint8:
        return A.e4m3_decode(raw) * w.kv_scale
    return A.bf16_decode(raw)


def test_e4m3_decode_every_code_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = A.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_single_key_returns_its_value():
    w = I.attn_custom(3, 16, 1)
    inp = I.make_attn_inputs(w)
    out = _run(w, inp)
    for b in range(3):
        assert np.array_equal(out[b], np.repeat(_rows(w, inp, b)[:, :512], 16, axis=0))


def test_repeated_key_returns_its_value():
    w = I.attn_custom(1, 16, 100, block_size=16)
    inp = I.make_attn_inputs(w)
    inp["cache"][:] = inp["cache"][inp["block_table"][0, 0], 5]
    out = _run(w, inp)
    v = A.bf16_decode(bits(inp["cache"][0, 0]))[:512]
    assert np.allclose(out[0], v[None, :], rtol=0, atol=1e-12)


def test_zero_query_averages_values():
    w = I.attn_custom(2, 4, (7, 130), block_size=16)
    inp = I.make_attn_inputs(w)
    inp["q"].zero_()
    out = _run(w, inp)
    for b in range(2):
        mean = _rows(w, inp, b)[:, :512].mean(axis=0)
        assert np.allclose(out[b], mean[None, :], rtol=1e-12, atol=1e-12)


def test_two_keys_closed_form():
    w = I.attn_custom(1, 8, 2)
    inp = I.make_attn_inputs(w, seed=5)
    out = _run(w, inp)
    q = A.bf16_decode(bits(inp["q"][0]))
    r = _rows(w, inp, 0)
    s = (q @ r.T) * w.sm_scale
    p0 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    want = p0[:, None] * r[0, :512] + (1.0 - p0[:, None]) * r[1, :512]
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-12)


def test_page_order_invariance():
    """Moving a sequence's pages elsewhere in the cache (and its block table
    with them) does not change the result."""
    w = I.attn_custom(2, 16, (200, 77), block_size=32)
    inp = I.make_attn_inputs(w, seed=6)
    out = _run(w, inp)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(1))
    moved = dict(inp)
    moved["cache"] = torch.empty_like(inp["cache"])
    moved["cache"][perm] = inp["cache"]
    moved["block_table"] = perm[inp["block_table"].long()].to(torch.int32)
    assert np.array_equal(_run(w, moved), out)


def test_score_shift_invariance():
    """A query component along a dimension in which every key is equal
    shifts all scores by one constant: the result does not change."""
    w = I.attn_custom(1, 16, 90)
    inp = I.make_attn_inputs(w, seed=7)
    inp["cache"][..., 570] = 1.0
    base = _run(w, inp)
    inp["q"][..., 570] += 3.0
    assert np.allclose(_run(w, inp), base, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("qf,kf", [(False, False), (False, True), (True, True)])
def test_matches_library_sdpa(qf, kf):
    w = I.attn_custom(3, 16, (1, 65, 300), q_fp8=qf, kv_fp8=kf)
    inp = I.make_attn_inputs(w, seed=8)
    out = _run(w, inp)
    qd = (torch.from_numpy(bits(inp["q"])).view(torch.float8_e4m3fn).double() * w.q_scale if qf
          else inp["q"].double())
    for b in range(3):
        rows = torch.from_numpy(_rows(w, inp, b))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qd[b][:, None, :], rows[None], rows[None, :, :512], scale=w.sm_scale)[:, 0, :]
        assert np.allclose(out[b], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_empty_sequence_gives_zeros():
    w = I.attn_custom(2, 16, (0, 5))
    inp = I.make_attn_inputs(w)
    out = _run(w, inp)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def _run_abs(w, inp):
    return A.mla_decode_attention(bits(inp["q"]), bits(inp["cache"]), inp["block_table"].numpy(),
                                  inp["seq_lens"].numpy(), w.sm_scale,
                                  w.q_scale if w.q_fp8 else None, w.kv_scale if w.kv_fp8 else None,
                                  with_abs=True)


def test_weighted_abs_single_key_and_zero_query():
    """sum_j p_j |v_j|: one key gives |v| exactly; a zero query (uniform
    weights) gives the mean of |v| over the sequence."""
    w = I.attn_custom(2, 16, 1, kv_fp8=True)
    inp = I.make_attn_inputs(w)
    out, mag = _run_abs(w, inp)
    assert np.array_equal(out, _run(w, inp))
    for b in range(2):
        assert np.array_equal(mag[b], np.abs(np.repeat(_rows(w, inp, b)[:, :512], 16, axis=0)))
    w = I.attn_custom(2, 4, (9, 150), block_size=16)
    inp = I.make_attn_inputs(w, seed=9)
    inp["q"].zero_()
    _, mag = _run_abs(w, inp)
    for b in range(2):
        want = np.abs(_rows(w, inp, b)[:, :512]).mean(axis=0)
        assert np.allclose(mag[b], want[None, :], rtol=1e-12, atol=0)


def test_weighted_abs_bounds_and_equality_for_nonnegative_values():
    """|out| <= sum_j p_j |v_j| <= max_j |v_j| (triangle inequality, weights
    summing to 1); with every value non-negative the two sums coincide."""
    w = I.attn_custom(3, 16, (1, 70, 600), kv_fp8=True)
    inp = I.make_attn_inputs(w, seed=10)
    out, mag = _run_abs(w, inp)
    assert np.all(np.abs(out) <= mag * (1 + 1e-12))
    for b in range(3):
        assert np.all(mag[b] <= np.abs(_rows(w, inp, b)[:, :512]).max(axis=0)[None, :] * (1 + 1e-12))
    assert np.any(np.abs(out) < 0.5 * mag)       # signs cancel in the plain sum
    raw = inp["cache"].view(torch.uint8)
    raw &= 0x7F                                  # clear every sign bit
    out, mag = _run_abs(w, inp)
    assert np.allclose(out, mag, rtol=1e-12, atol=0)
