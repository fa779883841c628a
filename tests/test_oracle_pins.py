"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a fact that the prhub summary of vLLM
PR #54896 (Kimi-K3 MLA decode kernel) or the mathematics fixes: the page's own
identity test (section "key source snippets"), the OCP E4M3 and IEEE bf16
format definitions (brute force over the code table, library casts, hand-derived
points in tests/golden/), and closed forms of the rotation (complex rotation,
norm preservation, relative-position invariance, exact hand rows).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mla_decode_concat_amd import inputs as I
from tests._util import bits, oracle_run

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


# ---------------------------------------------------------------- E4M3 ----

def _e4m3_code_values() -> np.ndarray:
    """Value of every code 0..255 from the OFP8 E4M3 layout (NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def _nearest_e4m3(x: np.ndarray) -> np.ndarray:
    """Brute force: nearest finite code to each value, ties to the even code,
    saturating at +-448, NaN -> S.1111.111."""
    vals = _e4m3_code_values()
    pos_codes = np.arange(0, 0x7F)             # +0 .. 448, ascending in value
    pos_vals = vals[pos_codes]
    assert np.all(np.diff(pos_vals) > 0)
    out = np.empty(x.shape, dtype=np.uint8)
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << 7
    idx = np.searchsorted(pos_vals, a, side="left")       # pos_vals[idx-1] < a <= pos_vals[idx]
    idx_hi = np.clip(idx, 0, len(pos_vals) - 1)
    idx_lo = np.clip(idx - 1, 0, len(pos_vals) - 1)
    d_hi = np.abs(pos_vals[idx_hi] - a)
    d_lo = np.abs(a - pos_vals[idx_lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (pos_codes[idx_lo] % 2 == 0))
    code = np.where(pick_lo, pos_codes[idx_lo], pos_codes[idx_hi])
    code = np.where(a >= 448.0, 0x7E, code)
    out[:] = code.astype(np.uint8) | sign
    out[np.isnan(x)] = 0x7F | sign[np.isnan(x)]
    return out


def test_e4m3_golden_points():
    g = _golden("e4m3_points.json")
    for p in g["encode"]:
        x = _f(p["x"])
        assert oracle.f32_to_e4m3(x) == int(p["code"], 16), p
    inv = float(np.float32(1.0) / np.float32(0.05))
    assert inv == 20.0
    for p in g["quantise_scale_0p05"]["points"]:
        assert oracle.quant_e4m3(p["x"], inv) == int(p["code"], 16), p


def test_e4m3_brute_force_wide_range():
    """Every fp32 exponent from 2^-12 to 2^9, a dense mantissa sample plus every
    midpoint between neighbouring codes and its two fp32 neighbours."""
    rng = np.random.default_rng(11)
    xs = []
    for e in range(-12, 10):
        m = rng.integers(0, 1 << 23, size=20000, dtype=np.int64)
        u = ((e + 127) << 23) | m
        xs.append(u.astype(np.uint32).view(np.float32))
    vals = _e4m3_code_values()[0:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2.0).astype(np.float32)
    xs.append(mids)
    xs.append(np.nextafter(mids, np.float32(np.inf)))
    xs.append(np.nextafter(mids, np.float32(0)))
    xs.append(vals.astype(np.float32))
    x = np.concatenate(xs).astype(np.float32)
    x = np.concatenate([x, -x])
    got = oracle.f32_to_e4m3_array(x)
    want = _nearest_e4m3(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("scale", [1.0, 0.05, 2.0 ** -4, 3.7])
def test_e4m3_exhaustive_bf16_vs_torch(scale):
    """All 65536 bf16 bit patterns, quantised under the scale, equal torch's
    library cast of the clamped product (torch's cast rounds to nearest even
    but does not saturate, hence the clamp); NaN compared as NaN."""
    b = np.arange(65536, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    got = oracle.quant_e4m3_array(x, scale)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (x * inv).astype(np.float32)
    v = torch.from_numpy(prod)
    want = torch.clamp(v, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(prod)
    assert np.all((got[nan] & 0x7F) == 0x7F)
    assert np.array_equal(got[~nan], want[~nan])


def test_e4m3_matches_brute_force_on_all_bf16():
    b = np.arange(65536, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    assert np.array_equal(oracle.f32_to_e4m3_array(x), _nearest_e4m3(x))


# ---------------------------------------------------------------- bf16 ----

def test_bf16_golden_points():
    g = _golden("bf16_points.json")
    for p in g["round"]:
        x = np.array([int(p["f32"], 16)], dtype=np.uint32).view(np.float32)
        assert oracle.f32_to_bf16_array(x)[0] == int(p["bf16"], 16), p
    for n in g["nan_inputs"]:
        x = np.array([int(n, 16)], dtype=np.uint32).view(np.float32)
        r = int(oracle.f32_to_bf16_array(x)[0])
        assert (r & 0x7F80) == 0x7F80 and (r & 0x7F) != 0


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and their neighbours
    hi = rng.integers(0, 1 << 16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16
    u = np.concatenate([u, hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    x = u.view(np.float32)
    got = oracle.f32_to_bf16_array(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_bf16_identity_on_exact_values():
    b = np.arange(65536, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    got = oracle.f32_to_bf16_array(x)
    ok = ~np.isnan(x)
    assert np.array_equal(got[ok], b[ok].astype(np.uint16))


# ---------------------------------------------------------------- fp16 ----

def test_fp16_golden_points():
    g = _golden("fp16_points.json")
    for p in g["round"]:
        x = np.array([_f(p["x"])], dtype=np.float32)
        assert oracle.f32_to_fp16_array(x)[0] == int(p["fp16"], 16), p


def test_fp16_rne_vs_numpy():
    """numpy's float32 -> float16 cast is IEEE round-to-nearest-even."""
    rng = np.random.default_rng(6)
    u = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    # dense coverage of the fp16 range, its ties and neighbours
    e = rng.integers(-26, 17, size=1_000_000)
    m = rng.random(1_000_000)
    y = (np.ldexp(1.0 + m, e) * np.where(rng.random(1_000_000) < 0.5, -1, 1)).astype(np.float32)
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    h = h[np.isfinite(h)]
    hs = np.unique(h)
    mids = ((hs[:-1] + hs[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, y, mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf))])
    got = oracle.f32_to_fp16_array(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_fp16_decode_all_patterns_vs_numpy():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f32_array(b)
    want = b.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ---------------------------------------------------------------- RoPE ----

def _x_bits(seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return bits((torch.randn(64, generator=g) * scale).to(torch.bfloat16))


def _f32(xb):
    return (xb.astype(np.uint32) << 16).view(np.float32)


def test_rope_golden_rows():
    g = _golden("rope_rows.json")
    x = np.array(g["x"], dtype=np.float32)
    xb = bits(torch.from_numpy(x).to(torch.bfloat16))
    assert np.array_equal(_f32(xb), x)       # inputs are bf16-exact
    for row in g["rows"]:
        cs = np.array([row["cos"]] * 32 + [row["sin"]] * 32, dtype=np.float32)
        y = oracle.rope_neox_f32(xb, cs)
        assert np.array_equal(y, np.array(row["y"], dtype=np.float32)), row["name"]


def test_gptj_rope_golden_rows():
    g = _golden("rope_rows.json")
    x = np.array(g["x"], dtype=np.float32)
    for row in g["rows_gptj"]:
        c = np.full(32, row["cos"], dtype=np.float32)
        s_ = np.full(32, row["sin"], dtype=np.float32)
        y = oracle.rope_f32(x, c, s_, gptj=True)
        assert np.array_equal(y, np.array(row["y"], dtype=np.float32)), row["name"]


def test_general_rotation_neox_matches_bf16_entry():
    table = I.rope_table(64).numpy()
    for seed in range(10):
        xb = _x_bits(900 + seed, scale=3.0)
        a = oracle.rope_neox_f32(xb, table[37])
        b = oracle.rope_f32(_f32(xb), table[37, :32], table[37, 32:], gptj=False)
        assert np.array_equal(a, b)


def test_gptj_rope_is_complex_rotation_by_position_angle():
    """Interleaved pairing as complex numbers: (x_2p + j x_2p+1) * exp(j pos
    theta^(-2p/64)), evaluated in float64 from the angle."""
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(7)
    p_idx = np.arange(32, dtype=np.float64)
    inv_freq = 10000.0 ** (-2.0 * p_idx / 64.0)
    for trial in range(200):
        pos = int(rng.integers(0, 4096))
        x = _f32(_x_bits(1100 + trial, scale=3.0))
        z = (x[0::2].astype(np.float64) + 1j * x[1::2]) * np.exp(1j * pos * inv_freq)
        want = np.empty(64)
        want[0::2], want[1::2] = z.real, z.imag
        got = oracle.rope_f32(x, table[pos, :32], table[pos, 32:], gptj=True).astype(np.float64)
        mag = np.abs(x[0::2]).astype(np.float64) + np.abs(x[1::2])
        tol = 3.0 * 2.0 ** -24 * np.repeat(mag, 2) + 1e-30
        assert np.all(np.abs(got - want) <= tol)


def test_gptj_rope_matches_library_rotate_every_two():
    table = I.rope_table(4096)
    rng = np.random.default_rng(8)
    for trial in range(100):
        pos = int(rng.integers(0, 4096))
        x = torch.from_numpy(_f32(_x_bits(1300 + trial, scale=4.0)).copy())
        cos = table[pos, :32].repeat_interleave(2)
        sin = table[pos, 32:].repeat_interleave(2)
        rot = torch.stack([-x[1::2], x[0::2]], dim=-1).reshape(64)
        want = (x * cos + rot * sin).numpy()
        got = oracle.rope_f32(x.numpy(), table[pos, :32].numpy(), table[pos, 32:].numpy(), gptj=True)
        assert np.array_equal(got, want)


def test_rope_position_zero_is_identity():
    table = I.rope_table(8)
    assert np.all(table[0, :32].numpy() == 1.0) and np.all(table[0, 32:].numpy() == 0.0)
    for seed in range(20):
        xb = _x_bits(seed, scale=10.0)
        y = oracle.rope_neox_f32(xb, table[0].numpy())
        assert np.array_equal(y, _f32(xb))


def test_rope_is_complex_rotation_by_position_angle():
    """NeoX pairing as complex numbers: (x_i + j x_{i+32}) * exp(j p theta^(-2i/64))
    evaluated in float64 from the angle itself (not the table)."""
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(1)
    i = np.arange(32, dtype=np.float64)
    inv_freq = 10000.0 ** (-2.0 * i / 64.0)
    for trial in range(200):
        p = int(rng.integers(0, 4096))
        xb = _x_bits(trial, scale=3.0)
        x = _f32(xb).astype(np.float64)
        z = (x[:32] + 1j * x[32:]) * np.exp(1j * p * inv_freq)
        want = np.concatenate([z.real, z.imag])
        got = oracle.rope_neox_f32(xb, table[p]).astype(np.float64)
        # fp32 table entries (rel 2^-24 each), two rounded products, one
        # rounded sum: bounded by 3 * 2^-24 * (|a| + |b|) per output
        mag = np.abs(x[:32]) + np.abs(x[32:])
        tol = 3.0 * 2.0 ** -24 * np.concatenate([mag, mag]) + 1e-30
        assert np.all(np.abs(got - want) <= tol), (p, np.max(np.abs(got - want) - tol))


def test_rope_f32_within_rounding_bound_of_f64():
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(2)
    for trial in range(200):
        p = int(rng.integers(0, 4096))
        xb = _x_bits(100 + trial, scale=5.0)
        y32 = oracle.rope_neox_f32(xb, table[p]).astype(np.float64)
        y64 = oracle.rope_neox_f64(xb, table[p])
        x = _f32(xb).astype(np.float64)
        c, s = table[p, :32].astype(np.float64), table[p, 32:].astype(np.float64)
        t1 = np.abs(x[:32] * c) + np.abs(x[32:] * s)
        t2 = np.abs(x[32:] * c) + np.abs(x[:32] * s)
        u = 2.0 ** -24
        bound = np.concatenate([t1, t2]) * (2 * u + u * u) + 1e-45
        assert np.all(np.abs(y32 - y64) <= bound)


@pytest.mark.parametrize("gptj", [False, True])
def test_rope_f64_is_the_complex_product_with_the_table_row(gptj):
    """The float64 twin (used by the rounding-bound pins) pairs the elements
    as the fp32 rotation does: as complex numbers (x_a + j x_b) times
    (cos + j sin) of the same table row, computed by numpy's complex product,
    with (a, b) = (i, i+32) or (2i, 2i+1)."""
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(12)
    for trial in range(100):
        p = int(rng.integers(0, 4096))
        x = _f32(_x_bits(1500 + trial, scale=3.0)).astype(np.float64)
        c, s = table[p, :32].astype(np.float64), table[p, 32:].astype(np.float64)
        a, b = (x[0::2], x[1::2]) if gptj else (x[:32], x[32:])
        z = (a + 1j * b) * (c + 1j * s)
        want = np.empty(64)
        if gptj:
            want[0::2], want[1::2] = z.real, z.imag
        else:
            want[:32], want[32:] = z.real, z.imag
        got = oracle.rope_f64(x.astype(np.float32), table[p, :32], table[p, 32:], gptj=gptj)
        mag = np.repeat(np.abs(a) + np.abs(b), 2) if gptj else np.concatenate([np.abs(a) + np.abs(b)] * 2)
        assert np.all(np.abs(got - want) <= 4 * 2.0 ** -53 * mag + 1e-300)


def test_gptj_rope_f32_within_rounding_bound_of_f64():
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(13)
    u = 2.0 ** -24
    for trial in range(200):
        p = int(rng.integers(0, 4096))
        x = _f32(_x_bits(1700 + trial, scale=5.0))
        y32 = oracle.rope_f32(x, table[p, :32], table[p, 32:], gptj=True).astype(np.float64)
        y64 = oracle.rope_f64(x, table[p, :32], table[p, 32:], gptj=True)
        a, b = x[0::2].astype(np.float64), x[1::2].astype(np.float64)
        c, s = table[p, :32].astype(np.float64), table[p, 32:].astype(np.float64)
        t = np.empty(64)
        t[0::2] = np.abs(a * c) + np.abs(b * s)
        t[1::2] = np.abs(b * c) + np.abs(a * s)
        assert np.all(np.abs(y32 - y64) <= t * (2 * u + u * u) + 1e-45)


def test_rope_matches_library_rotate_half_fp32():
    """Eager torch fp32: x*cos + rotate_half(x)*sin, each op rounded."""
    table = I.rope_table(4096)
    rng = np.random.default_rng(3)
    for trial in range(100):
        p = int(rng.integers(0, 4096))
        xb = _x_bits(300 + trial, scale=4.0)
        x = torch.from_numpy(_f32(xb).copy())
        cos = torch.cat([table[p, :32], table[p, :32]])
        sin = torch.cat([table[p, 32:], table[p, 32:]])
        rot = torch.cat([-x[32:], x[:32]])
        want = (x * cos + rot * sin).numpy()
        got = oracle.rope_neox_f32(xb, table[p].numpy())
        assert np.array_equal(got, want)


def test_rope_preserves_pair_norms_and_relative_position():
    table = I.rope_table(4096).numpy()
    rng = np.random.default_rng(4)
    for trial in range(50):
        xa, xk = _x_bits(500 + trial), _x_bits(700 + trial)
        p1, p2 = int(rng.integers(0, 2000)), int(rng.integers(0, 2000))
        d = int(rng.integers(1, 2000))
        ya = oracle.rope_neox_f64(xa, table[p1])
        x = _f32(xa).astype(np.float64)
        assert np.allclose(ya[:32] ** 2 + ya[32:] ** 2, x[:32] ** 2 + x[32:] ** 2, rtol=1e-6, atol=1e-12)
        dot1 = ya @ oracle.rope_neox_f64(xk, table[p2])
        dot2 = oracle.rope_neox_f64(xa, table[p1 + d]) @ oracle.rope_neox_f64(xk, table[p2 + d])
        assert abs(dot1 - dot2) <= 1e-5 * (1 + abs(dot1))


# ---------------------------------------------------------- whole epilogue ----

@pytest.mark.parametrize("num_tokens", [64, 65])
def test_page_identity_concat_and_scatter(num_tokens):
    """The page's own boundary test: with rotation and FP8 off, q equals
    cat(ql_nope, q_pe), the cache rows at the slots equal cat(kv_c, k_pe),
    and every other cache byte keeps its initial zero."""
    w = I.custom(num_tokens, 16, rope=False)
    inp = I.make_inputs(w)
    q, cache = oracle_run(w, inp)
    want_q = bits(torch.cat([inp["ql_nope"], inp["q_pe"]], dim=-1))
    assert np.array_equal(q, want_q)
    rows = cache.reshape(-1, 576)
    slots = inp["slot_mapping"].numpy()
    assert np.array_equal(rows[slots], bits(torch.cat([inp["kv_c"], inp["k_pe"]], dim=-1)))
    untouched = np.ones(rows.shape[0], dtype=bool)
    untouched[slots] = False
    assert np.all(rows[untouched] == 0)


def _torch_textbook(w, inp):
    """Library composition: cat, eager fp32 rotate_half / rotate_every_two
    rotation, activation-type cast or clamp + float8_e4m3fn cast.  Used only
    to pin the oracle."""
    pe_q = inp["q_pe"].float()
    pe_k = inp["k_pe"].float()
    act = w.torch_dtype
    if w.rope:
        cs = inp["rope_cos_sin"].float()[inp["positions"].clamp(0, w.max_position - 1)]
        if w.rope_style == "gptj":
            cos = cs[:, :32].repeat_interleave(2, dim=-1)
            sin = cs[:, 32:].repeat_interleave(2, dim=-1)

            def rot(x, c, s):
                r = torch.stack([-x[..., 1::2], x[..., 0::2]], dim=-1).reshape(x.shape)
                return x * c + r * s
        else:
            cos = torch.cat([cs[:, :32], cs[:, :32]], dim=-1)
            sin = torch.cat([cs[:, 32:], cs[:, 32:]], dim=-1)

            def rot(x, c, s):
                return x * c + torch.cat([-x[..., 32:], x[..., :32]], dim=-1) * s
        pe_q = rot(pe_q, cos[:, None, :], sin[:, None, :])
        pe_k = rot(pe_k, cos, sin)

    def enc(nope, pe_f32, fp8, scale):
        if fp8:
            inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
            v = torch.cat([nope.float(), pe_f32], dim=-1) * inv
            return bits(torch.clamp(v, -448, 448).to(torch.float8_e4m3fn))
        return bits(torch.cat([nope, pe_f32.to(act)], dim=-1))
    q = enc(inp["ql_nope"], pe_q, w.q_fp8, w.q_scale)
    kv = enc(inp["kv_c"], pe_k, w.kv_fp8, w.kv_scale)
    return q, kv


@pytest.mark.parametrize("name", ["t1_h16_copy", "t64_h16_rope_fp8", "t65_h16_rope_fp8"])
def test_oracle_matches_library_composition(name):
    w = I.WORKLOADS[name]
    inp = I.make_inputs(w)
    q, cache = oracle_run(w, inp)
    want_q, want_kv = _torch_textbook(w, inp)
    assert np.array_equal(q, want_q)
    rows = cache.reshape(-1, 576)
    assert np.array_equal(rows[inp["slot_mapping"].numpy()], want_kv)


@pytest.mark.parametrize("flags", [(True, False, False), (True, False, True), (True, True, False),
                                   (False, True, True), (False, False, True)])
def test_oracle_matches_library_composition_all_modes(flags):
    rope, qf, kf = flags
    w = I.custom(37, 5, num_blocks=3, rope=rope, q_fp8=qf, kv_fp8=kf, q_scale=0.03, kv_scale=0.2)
    inp = I.make_inputs(w, seed=9)
    q, cache = oracle_run(w, inp)
    want_q, want_kv = _torch_textbook(w, inp)
    assert np.array_equal(q, want_q)
    assert np.array_equal(cache.reshape(-1, 576)[inp["slot_mapping"].numpy()], want_kv)


@pytest.mark.parametrize("dtype,style,table", [("fp16", "neox", "f32"), ("bf16", "gptj", "f32"),
                                               ("bf16", "neox", "bf16"), ("fp16", "gptj", "bf16")])
@pytest.mark.parametrize("qf,kf", [(False, False), (True, False), (False, True), (True, True)])
def test_oracle_matches_library_composition_variants(dtype, style, table, qf, kf):
    w = I.custom(29, 3, num_blocks=2, rope=True, q_fp8=qf, kv_fp8=kf, q_scale=0.03, kv_scale=0.2,
                 dtype=dtype, rope_style=style, table_dtype=table)
    inp = I.make_inputs(w, seed=10)
    q, cache = oracle_run(w, inp)
    want_q, want_kv = _torch_textbook(w, inp)
    assert np.array_equal(q, want_q)
    assert np.array_equal(cache.reshape(-1, 576)[inp["slot_mapping"].numpy()], want_kv)


def test_fp16_copy_path_is_identity():
    w = I.custom(40, 4, num_blocks=1, dtype="fp16")
    inp = I.make_inputs(w, seed=12)
    q, cache = oracle_run(w, inp)
    assert np.array_equal(q, bits(torch.cat([inp["ql_nope"], inp["q_pe"]], dim=-1)))
    rows = cache.reshape(-1, 576)
    assert np.array_equal(rows[inp["slot_mapping"].numpy()],
                          bits(torch.cat([inp["kv_c"], inp["k_pe"]], dim=-1)))


def test_row_independence_prefix_property():
    """Rows do not interact: the first 64 tokens of a 65-token call equal a
    64-token call on the same inputs (the page's 64/65 boundary)."""
    w65 = I.WORKLOADS["t65_h16_rope_fp8"]
    inp = I.make_inputs(w65)
    q65, c65 = oracle_run(w65, inp)
    w64 = I.custom(64, 16, num_blocks=2, rope=True, q_fp8=True, kv_fp8=True)
    inp64 = {k: (v[:64] if k in ("ql_nope", "q_pe", "kv_c", "k_pe", "slot_mapping", "positions") else v)
             for k, v in inp.items()}
    inp64 = {k: (v.contiguous() if isinstance(v, torch.Tensor) else v) for k, v in inp64.items()}
    q64, c64 = oracle_run(w64, inp64)
    assert np.array_equal(q65[:64], q64)
    s65 = inp["slot_mapping"][64].item()
    r65, r64 = c65.reshape(-1, 576).copy(), c64.reshape(-1, 576)
    r65[s65] = 0
    assert np.array_equal(r65, r64)


def test_out_of_range_slots_leave_cache_untouched():
    w = I.custom(6, 2, num_blocks=1, rope=True, kv_fp8=True)
    inp = I.make_inputs(w, seed=4)
    inp["slot_mapping"] = torch.tensor([-1, 64, 3, 1 << 40, -7, 63], dtype=torch.int64)
    init = np.full((1, 64, 576), 0x5A, dtype=np.uint8)
    q, cache = oracle_run(w, inp, cache_init=init)
    rows = cache.reshape(-1, 576)
    changed = np.nonzero(np.any(rows != 0x5A, axis=1))[0]
    assert set(changed.tolist()) <= {3, 63}
    assert np.any(rows[3] != 0x5A) and np.any(rows[63] != 0x5A)


def test_positions_clamped_into_table():
    w = I.custom(3, 2, num_blocks=1, rope=True, max_position=16)
    inp = I.make_inputs(w, seed=8)
    inp["positions"] = torch.tensor([-5, 16, 1000], dtype=torch.int64)
    q, _ = oracle_run(w, inp)
    inp2 = dict(inp)
    inp2["positions"] = torch.tensor([0, 15, 15], dtype=torch.int64)
    q2, _ = oracle_run(w, inp2)
    assert np.array_equal(q, q2)


def test_duplicate_slots_keep_later_token():
    w = I.custom(3, 1, num_blocks=1)
    inp = I.make_inputs(w, seed=2)
    inp["slot_mapping"] = torch.tensor([5, 5, 9], dtype=torch.int64)
    _, cache = oracle_run(w, inp)
    want = bits(torch.cat([inp["kv_c"][1], inp["k_pe"][1]]))
    assert np.array_equal(cache.reshape(-1, 576)[5], want)


# ------------------------------------------- the absorbed key projection ----
# The product that produces ql_nope (the page's kernel reads its output,
# "implementation breakdown" item 2): ql[t,h,n] = sum_k q_nope[t,h,k] W_UK[h,k,n],
# with W_UK handed over transposed as w_uk_t[h,n,k].

def _act(x: torch.Tensor, fp16: bool) -> np.ndarray:
    dt = torch.float16 if fp16 else torch.bfloat16
    return x.to(dt).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fp16", [False, True])
def test_uk_product_matches_library_matmul(fp16):
    """A float64 matmul of the decoded values, per head (library routine)."""
    g = torch.Generator().manual_seed(11)
    T, H = 9, 3
    q = _act(torch.randn(T, H, 128, generator=g), fp16)
    w = _act(torch.randn(H, 512, 128, generator=g) * 128 ** -0.5, fp16)
    dt = torch.float16 if fp16 else torch.bfloat16
    qd = torch.from_numpy(q.view(np.int16)).view(dt).double().numpy()
    wd = torch.from_numpy(w.view(np.int16)).view(dt).double().numpy()
    ref = np.stack([qd[:, h, :] @ wd[h].T for h in range(H)], axis=1)
    ql, mag = oracle.uk_product(q, w, fp16=fp16, with_mag=True)
    np.testing.assert_allclose(ql, ref, rtol=1e-13, atol=1e-13)
    ref_mag = np.stack([np.abs(qd[:, h, :]) @ np.abs(wd[h]).T for h in range(H)], axis=1)
    np.testing.assert_allclose(mag, ref_mag, rtol=1e-13, atol=0)


def test_uk_product_unit_rows_select_one_input():
    """Row n of head h's transposed weight is the unit vector e_{(5n + 3h) % 128}:
    the product then picks q_nope[t, h, (5n + 3h) % 128] exactly.  A transposed
    weight, a wrong head or a shifted k fails this."""
    g = torch.Generator().manual_seed(12)
    T, H = 4, 5
    q = _act(torch.randn(T, H, 128, generator=g), False)
    w = np.zeros((H, 512, 128), dtype=np.uint16)
    pick = np.array([[(5 * n + 3 * h) % 128 for n in range(512)] for h in range(H)])
    for h in range(H):
        w[h, np.arange(512), pick[h]] = 0x3F80           # bf16 1.0
    ql, mag = oracle.uk_product(q, w, with_mag=True)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    for h in range(H):
        assert np.array_equal(ql[:, h, :], qd[:, h, pick[h]])
        assert np.array_equal(mag[:, h, :], np.abs(qd[:, h, pick[h]]))


def test_uk_product_integers_brute_force():
    """Small integers (exact in bf16) against an integer triple loop."""
    rng = np.random.default_rng(13)
    T, H = 2, 2
    qi = rng.integers(-8, 9, size=(T, H, 128))
    wi = rng.integers(-8, 9, size=(H, 512, 128))
    q = _act(torch.from_numpy(qi).float(), False)
    w = _act(torch.from_numpy(wi).float(), False)
    ql, mag = oracle.uk_product(q, w, with_mag=True)
    for t in range(T):
        for h in range(H):
            for n in range(0, 512, 37):
                exact = sum(int(qi[t, h, k]) * int(wi[h, n, k]) for k in range(128))
                absum = sum(abs(int(qi[t, h, k]) * int(wi[h, n, k])) for k in range(128))
                assert ql[t, h, n] == exact and mag[t, h, n] == absum


def test_uk_product_magnitude_is_the_absolute_sum():
    """Nonnegative inputs: the absolute sum equals the sum; flipping signs
    leaves it and only shrinks the sum."""
    g = torch.Generator().manual_seed(14)
    qa = torch.rand(3, 2, 128, generator=g)
    wa = torch.rand(2, 512, 128, generator=g)
    ql, mag = oracle.uk_product(_act(qa, False), _act(wa, False), with_mag=True)
    assert np.array_equal(ql, mag)
    sign = torch.where(torch.rand(3, 2, 128, generator=g) < 0.5, -1.0, 1.0)
    ql2, mag2 = oracle.uk_product(_act(qa * sign, False), _act(wa, False), with_mag=True)
    assert np.array_equal(mag2, mag) and np.all(np.abs(ql2) <= mag2)
