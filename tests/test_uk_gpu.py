"""GPU parity of the epilogue fused into the W_UK product
(mla_decode_uk_q_concat_kv_insert, include/mla_dq.h) against the oracle.

Bar:
  * q_out's latent columns.  The kernel forms each one as an fp32 sum of the
    128 exact products q_nope[t,h,k] * W_UK[h,k,n] in its own order of
    additions, then encodes that fp32 value once.  The oracle gives the exact
    sum x and the sum of absolute products m (fp64).  Every stored code must
    lie, as a value, between enc(fl32(x - e)) and enc(fl32(x + e)) with
    e = 2^-16 * m (twice the worst-case rounding error of a 128-term fp32
    sum), enc being the oracle's bf16 / fp16 rounding or its E4M3
    quantisation under q_scale; both are monotone, and any fp32 value within
    e of x rounds into that range.  At least 99 % of the codes must equal
    enc(fl32(x)) exactly.
  * q_out's positional tails and the whole cache: bit-exact against the
    oracle's epilogue (they do not depend on the product).
Guard bands around q_out and the cache catch stray writes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mla_decode_concat_amd as M
from mla_decode_concat_amd import inputs as I
import oracle
from tests._util import bits, oracle_run
from tests.test_gpu_parity import GUARD_ROWS, _background, _out_of_range, announce, assert_same, flags_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_BOUND = 2.0 ** -16
MIN_EXACT = 0.99


def run_uk(w: I.Workload, inp: dict, extra_flags: int = 0, cache_init: np.ndarray | None = None,
           contiguous: bool = False, case: str = ""):
    """Run the fused kernel on device copies of inp; returns (q bits, cache bits)."""
    announce(f"uk {case} {w.describe()} flags+{extra_flags:#x}{' contiguous' if contiguous else ''}")
    T, H = w.tokens, w.heads
    qdt = torch.float8_e4m3fn if w.q_fp8 else w.torch_dtype
    kvdt = torch.float8_e4m3fn if w.kv_fp8 else w.torch_dtype
    n_q = T * H * I.ROW
    pad = 4096
    qbig = torch.empty(n_q + 2 * pad, dtype=qdt, device=DEV)
    qbig.view(torch.uint8).fill_(0xFF)
    q_out = qbig[pad:pad + n_q].view(T, H, I.ROW)
    if cache_init is None:
        cache_cpu = inp["cache"]
    else:
        cache_cpu = torch.from_numpy(cache_init.view(np.int16 if cache_init.dtype == np.uint16 else np.uint8)
                                     .copy()).view(kvdt)
    NB, BS = cache_cpu.shape[0], cache_cpu.shape[1]
    cbig = torch.empty(NB + 2 * GUARD_ROWS, BS, I.ROW, dtype=kvdt, device=DEV)
    gen = torch.Generator().manual_seed(4321)
    guard = torch.randint(0, 256, (GUARD_ROWS, BS, I.ROW * cbig.element_size()), generator=gen,
                          dtype=torch.uint8)
    cbig.view(torch.uint8)[:GUARD_ROWS] = guard.to(DEV)
    cbig.view(torch.uint8)[-GUARD_ROWS:] = guard.to(DEV)
    cache = cbig[GUARD_ROWS:GUARD_ROWS + NB]
    cache.copy_(cache_cpu.to(DEV))
    q_b = inp["q_b"].to(DEV)
    q_nope, q_pe = q_b[..., :I.UK_K], q_b[..., I.UK_K:]
    if contiguous:
        q_nope, q_pe = q_nope.contiguous(), q_pe.contiguous()
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()
           if k not in ("q_b", "q_nope", "q_pe")}
    M.mla_decode_uk_q_concat_kv_insert(q_out, q_nope, dev["w_uk_t"], q_pe, dev["kv_c"], dev["k_pe"], cache,
                                       dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"],
                                       dev["q_scale"], dev["kv_scale"], flags_of(w) | extra_flags)
    torch.cuda.synchronize()
    qb = qbig.view(torch.uint8).cpu()
    assert torch.all(qb[:pad * qbig.element_size()] == 0xFF), "write before q_out"
    assert torch.all(qb[(pad + n_q) * qbig.element_size():] == 0xFF), "write after q_out"
    cb = cbig.view(torch.uint8).cpu()
    assert torch.equal(cb[:GUARD_ROWS], guard) and torch.equal(cb[-GUARD_ROWS:], guard), \
        "write outside the cache"
    return bits(q_out.cpu()), bits(cache.cpu())


def _encode(v32: np.ndarray, w: I.Workload) -> np.ndarray:
    """The oracle's encoding of fp32 latent values into q_out codes."""
    if w.q_fp8:
        return oracle.quant_e4m3_array(v32, w.q_scale).reshape(v32.shape)
    if w.dtype == "fp16":
        return oracle.f32_to_fp16_array(v32).reshape(v32.shape)
    return oracle.f32_to_bf16_array(v32).reshape(v32.shape)


def _value(codes: np.ndarray, w: I.Workload) -> np.ndarray:
    if w.q_fp8:
        return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()
    if w.dtype == "fp16":
        return codes.view(np.float16).astype(np.float32)
    return (codes.astype(np.uint32) << 16).view(np.float32)


def check_latent(got: np.ndarray, q_nope_bits: np.ndarray, w_bits: np.ndarray, w: I.Workload,
                 what: str = "q latent") -> float:
    """The bar on q_out[..., :512] (see the module docstring); returns the
    fraction of codes equal to enc(fl32(x))."""
    x, mag = oracle.uk_product(q_nope_bits, w_bits, fp16=w.dtype == "fp16", with_mag=True)
    e = REL_BOUND * mag
    lo = _value(_encode((x - e).astype(np.float32), w), w)
    hi = _value(_encode((x + e).astype(np.float32), w), w)
    mid = _encode(x.astype(np.float32), w)
    g = _value(got, w)
    bad = np.nonzero(~((lo <= g) & (g <= hi)))
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} codes outside the bound, first at {i}: got {g[i]!r}, "
                             f"allowed [{lo[i]!r}, {hi[i]!r}], exact sum {x[i]!r}")
    exact = float(np.mean(got == mid))
    assert exact >= MIN_EXACT, f"{what}: only {exact:.4f} of the codes equal enc(fl32(exact sum))"
    return exact


def expected_rest(w: I.Workload, inp: dict, cache_init=None):
    """The oracle's tails and cache (any ql_nope: the latent part is checked apart)."""
    epi = dict(inp)
    epi["ql_nope"] = torch.zeros(w.tokens, w.heads, I.NOPE, dtype=w.torch_dtype)
    return oracle_run(w, epi, cache_init=cache_init)


def check_all(w: I.Workload, inp: dict, q, cache, cache_init=None) -> float:
    want_q, want_cache = expected_rest(w, inp, cache_init)
    fp16 = w.dtype == "fp16"
    assert_same(q[..., I.NOPE:], want_q[..., I.NOPE:], "q tails", fp16)
    assert_same(cache, want_cache, "cache", fp16)
    return check_latent(q[..., :I.NOPE], bits(inp["q_nope"]), bits(inp["w_uk_t"]), w)


def workload(T, H, rope=True, q_fp8=False, kv_fp8=True, **kw) -> I.Workload:
    return I.custom(T, H, rope=rope, q_fp8=q_fp8, kv_fp8=kv_fp8, name="uk", **kw)


MODES = [(r, q, k) for r in (False, True) for q in (False, True) for k in (False, True)]
SHAPES = [(1, 16), (5, 16), (16, 16), (17, 16), (64, 16), (65, 16), (128, 16), (255, 16),
          (1, 128), (64, 128), (3, 1), (40, 3), (300, 5)]


@pytest.mark.parametrize("T,H", SHAPES, ids=[f"t{t}_h{h}" for t, h in SHAPES])
@pytest.mark.parametrize("mode", [(True, False, True), (True, True, True)], ids=["q_bf16_kv_e4m3", "q_kv_e4m3"])
def test_uk_shapes(T, H, mode):
    w = workload(T, H, *mode)
    inp = I.make_uk_inputs(w)
    q, cache = run_uk(w, inp, case=f"shape t{T} h{H}")
    check_all(w, inp, q, cache)


@pytest.mark.parametrize("mode", MODES, ids=[f"rope{int(r)}_q{int(q)}_kv{int(k)}" for r, q, k in MODES])
@pytest.mark.parametrize("T,H", [(65, 16), (255, 16)], ids=["t65_h16", "t255_h16"])
def test_uk_all_modes(T, H, mode):
    w = workload(T, H, *mode)
    inp = I.make_uk_inputs(w)
    q, cache = run_uk(w, inp, case="modes")
    check_all(w, inp, q, cache)


FORCED = [("small", M.FORCE_SMALL_T), ("large", M.FORCE_LARGE_T),
          ("small_stream", M.FORCE_SMALL_T | M.FORCE_STREAM), ("large_stream", M.FORCE_LARGE_T | M.FORCE_STREAM),
          ("large_cached", M.FORCE_LARGE_T | M.FORCE_CACHED)]


@pytest.mark.parametrize("name,extra", FORCED, ids=[f[0] for f in FORCED])
@pytest.mark.parametrize("T,H", [(1, 16), (65, 16), (300, 5), (1000, 16), (97, 128)],
                         ids=["t1_h16", "t65_h16", "t300_h5", "t1000_h16", "t97_h128"])
def test_uk_forced_configurations(T, H, name, extra):
    w = workload(T, H, True, True, True)
    inp = I.make_uk_inputs(w)
    p = M.uk_plan(M._binding._dims(inp["q_nope"], inp["q_pe"], inp["kv_c"], inp["k_pe"], inp["cache"],
                                   inp["rope_cos_sin"]), flags_of(w) | extra)
    assert p.mapping == (0 if "small" in name else 1)
    q, cache = run_uk(w, inp, extra, case=name)
    check_all(w, inp, q, cache)


VARIANTS = [("fp16", dict(dtype="fp16")), ("gptj", dict(rope_style="gptj")),
            ("table_bf16", dict(table_dtype="bf16")),
            ("fp16_gptj_table_bf16", dict(dtype="fp16", rope_style="gptj", table_dtype="bf16"))]


@pytest.mark.parametrize("name,kw", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("mode", [(True, False, False), (True, True, True)], ids=["unquantised", "e4m3"])
@pytest.mark.parametrize("T,H", [(65, 16), (300, 5)], ids=["t65_h16", "t300_h5"])
def test_uk_variants(T, H, mode, name, kw):
    w = workload(T, H, *mode, **kw)
    inp = I.make_uk_inputs(w)
    for extra in (0, M.FORCE_LARGE_T):
        q, cache = run_uk(w, inp, extra, case=name)
        check_all(w, inp, q, cache)


@pytest.mark.parametrize("T,H", [(64, 16), (300, 5)], ids=["t64_h16", "t300_h5"])
def test_uk_contiguous_inputs(T, H):
    w = workload(T, H, True, True, True)
    inp = I.make_uk_inputs(w)
    q, cache = run_uk(w, inp, contiguous=True, case="contiguous")
    check_all(w, inp, q, cache)


@pytest.mark.parametrize("T,H", [(70, 16), (40, 3), (200, 1)], ids=["t70_h16", "t40_h3", "t200_h1"])
@pytest.mark.parametrize("name,extra", [("plan", 0), ("small", M.FORCE_SMALL_T), ("large", M.FORCE_LARGE_T),
                                        ("large_stream", M.FORCE_LARGE_T | M.FORCE_STREAM)],
                         ids=["plan", "small", "large", "large_stream"])
def test_uk_junk_slots_positions_and_background(T, H, name, extra):
    """Padding slots (-1), slots past the cache, positions outside the table
    and a random cache background, under both configurations (the
    throughput one stages the table rows of its tail workgroups, clamped, in
    LDS): skipped rows keep their bytes."""
    w = workload(T, H, True, True, True, num_blocks=(T + 63) // 64 + 2)
    inp = I.make_uk_inputs(w)
    slots = inp["slot_mapping"].clone()
    slots[::7] = -1
    slots[3] = w.num_slots + 5
    slots[4] = -(1 << 40)
    inp["slot_mapping"] = slots
    pos = inp["positions"].clone()
    pos[::5] = -3
    pos[2] = w.max_position + 10
    inp["positions"] = pos
    rng = np.random.default_rng(5)
    cache_init = rng.integers(0, 256, size=(w.num_blocks, w.block_size, I.ROW), dtype=np.uint8)
    cache_init[(cache_init & 0x7F) == 0x7F] = 0    # no NaN codes in the background
    q, cache = run_uk(w, inp, extra, cache_init=cache_init, case=f"junk {name}")
    check_all(w, inp, q, cache, cache_init=cache_init)


@pytest.mark.parametrize("T,H", [(3, 2), (120, 3)], ids=["t3_h2", "t120_h3"])
@pytest.mark.parametrize("name,extra", [("small", M.FORCE_SMALL_T), ("large", M.FORCE_LARGE_T),
                                        ("large_stream", M.FORCE_LARGE_T | M.FORCE_STREAM)],
                         ids=["small", "large", "large_stream"])
def test_uk_duplicate_slots_leave_one_candidate(T, H, name, extra):
    """Tokens that share a slot: every 8-element chunk of that cache row comes
    from one of them (the header's contract); q_out and the rows of unique
    slots meet the bar, under both configurations."""
    w = workload(T, H, True, True, True, num_blocks=(T + 63) // 64 + 1, kv_scale=0.3)
    inp = I.make_uk_inputs(w, seed=2 + T)
    slots = inp["slot_mapping"].numpy().copy()
    groups = [[0, 1]] if T == 3 else [[0, 1, 2], [5, 60], [33, 119, 64, 90]]
    for g in groups:
        slots[g] = slots[g[0]]
    inp["slot_mapping"] = torch.from_numpy(slots)
    q, cache = run_uk(w, inp, extra, case=f"duplicate slots {name}")
    want_q, want_cache = expected_rest(w, inp)
    assert_same(q[..., I.NOPE:], want_q[..., I.NOPE:], "q tails")
    check_latent(q[..., :I.NOPE], bits(inp["q_nope"]), bits(inp["w_uk_t"]), w)
    rows, want_rows = cache.reshape(-1, I.ROW), want_cache.reshape(-1, I.ROW)
    shared = {int(slots[g[0]]): g for g in groups}
    keep = np.ones(rows.shape[0], dtype=bool)
    keep[list(shared)] = False
    assert_same(rows[keep], want_rows[keep], "cache rows of unique slots and untouched rows")
    w1 = workload(1, H, True, True, True, num_blocks=1, kv_scale=0.3)
    for s_, g in shared.items():
        cands = []
        for t in g:       # the row token t alone would write
            sub = dict(inp, slot_mapping=torch.tensor([0], dtype=torch.int64),
                       cache=torch.zeros(1, 64, I.ROW, dtype=torch.float8_e4m3fn),
                       ql_nope=torch.zeros(1, H, I.NOPE, dtype=w.torch_dtype))
            for k in ("q_pe", "kv_c", "k_pe", "positions"):
                sub[k] = inp[k][t:t + 1].clone()
            cands.append(oracle_run(w1, sub)[1].reshape(-1, I.ROW)[0].reshape(72, 8))
        got = rows[s_].reshape(72, 8)
        for c in range(72):
            assert any(np.array_equal(got[c], cand[c]) for cand in cands), (s_, c)


def _random_uk_case(i: int):
    """Seeded random shape and mode of the fused call: tokens, heads, block
    size, precision of each output, activation type, rotation style and table
    type, launch override, q_nope strided or contiguous, share of padding and
    out-of-range slots and positions, and a random cache background."""
    rng = np.random.default_rng(2000 + i)
    H = int(rng.choice([1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 64, 65, 128]))
    T = int(rng.integers(1, max(2, min(2000, 24000 // H))))
    bs = int(rng.choice([1, 16, 64, 128]))
    rope, qf, kf = bool(rng.integers(2)), bool(rng.integers(2)), bool(rng.integers(2))
    dtype = "fp16" if rng.integers(4) == 0 else "bf16"
    style = "gptj" if rope and rng.integers(3) == 0 else "neox"
    table = "bf16" if rope and rng.integers(3) == 0 else "f32"
    nb = (T + bs - 1) // bs + int(rng.integers(0, 3))
    force = [0, M.FORCE_SMALL_T, M.FORCE_LARGE_T, M.FORCE_SMALL_T | M.FORCE_STREAM,
             M.FORCE_LARGE_T | M.FORCE_STREAM, M.FORCE_LARGE_T | M.FORCE_CACHED][int(rng.integers(6))]
    w = workload(T, H, rope, qf, kf, num_blocks=nb, block_size=bs,
                 q_scale=float(rng.choice([0.05, 0.3, 1.0])), kv_scale=float(rng.choice([0.05, 2.0])),
                 dtype=dtype, rope_style=style, table_dtype=table,
                 max_position=int(rng.choice([1, 77, 4096])))
    junk = float(rng.choice([0.0, 0.0, 0.1, 0.5]))
    return w, force, int(rng.integers(1 << 30)), junk, bool(rng.integers(2)), bool(rng.integers(2))


@pytest.mark.parametrize("i", range(24))
def test_uk_seeded_random_shapes_and_modes(i):
    """Random shapes, heads, block sizes, flag and variant combinations and
    launch overrides of the fused call, some with padding or out-of-range
    slots and positions over a random cache background, each against the
    oracle to the bar above."""
    w, force, seed, junk, contiguous, background = _random_uk_case(i)
    inp = I.make_uk_inputs(w, seed=seed)
    if junk:
        inp = _out_of_range(inp, w, seed=seed + 1, frac=junk)
    cache_init = _background(w, seed + 2) if background else None
    q, cache = run_uk(w, inp, force, cache_init=cache_init, contiguous=contiguous,
                      case=f"random case {i} (seed {seed}, junk {junk})")
    check_all(w, inp, q, cache, cache_init=cache_init)


def test_uk_e4m3_saturation():
    """A small q_scale drives most latent values past 448: they saturate."""
    w = workload(33, 16, True, True, True, q_scale=0.002)
    inp = I.make_uk_inputs(w)
    q, cache = run_uk(w, inp, case="saturation")
    check_all(w, inp, q, cache)
    assert np.mean((q[..., :I.NOPE] & 0x7F) == 0x7E) > 0.3


def test_uk_zero_tokens():
    w = workload(4, 16, True, True, True)
    inp = I.make_uk_inputs(w)
    T0 = {k: (v[:0] if k in ("q_b", "q_nope", "q_pe", "kv_c", "k_pe", "slot_mapping", "positions") else v)
          for k, v in inp.items()}
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in T0.items()}
    q_out = torch.empty(0, 16, I.ROW, dtype=torch.float8_e4m3fn, device=DEV)
    cache = dev["cache"].clone()
    M.mla_decode_uk_q_concat_kv_insert(q_out, dev["q_nope"], dev["w_uk_t"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                       cache, dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"],
                                       dev["q_scale"], dev["kv_scale"], flags_of(w))
    torch.cuda.synchronize()
    assert torch.equal(cache.cpu().view(torch.uint8), inp["cache"].view(torch.uint8))


@pytest.mark.parametrize("T,H,mode", [(256, 128, (True, True, False)), (8192, 16, (True, False, True))],
                         ids=["t256_h128_q_e4m3_kv_bf16", "t8192_h16_q_bf16_kv_e4m3"])
def test_uk_full_size(T, H, mode):
    """The two large decode shapes under the default plan: tails and cache in
    full, the latent columns of a sample of tokens (every token's range
    boundary region and the last tokens included)."""
    num_blocks = (T + 63) // 64 + 1
    w = workload(T, H, *mode, num_blocks=num_blocks)
    inp = I.make_uk_inputs(w)
    q, cache = run_uk(w, inp, case="full size")
    want_q, want_cache = expected_rest(w, inp)
    assert_same(q[..., I.NOPE:], want_q[..., I.NOPE:], "q tails")
    assert_same(cache, want_cache, "cache")
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([np.arange(0, min(T, 48)), np.arange(max(0, T - 48), T),
                                       np.arange(112, T, 128), np.arange(127, T, 128),
                                       rng.choice(T, size=min(T, 256), replace=False)]))
    check_latent(q[sample, :, :I.NOPE], bits(inp["q_nope"])[sample], bits(inp["w_uk_t"]), w)


ALL_LAUNCHES = [("plan", 0), ("small_cached", M.FORCE_SMALL_T | M.FORCE_CACHED),
                ("small_stream", M.FORCE_SMALL_T | M.FORCE_STREAM),
                ("large_cached", M.FORCE_LARGE_T | M.FORCE_CACHED),
                ("large_stream", M.FORCE_LARGE_T | M.FORCE_STREAM)]


@pytest.mark.parametrize("T,H,mode", [(1, 16, (True, True, True)), (33, 16, (True, True, True)),
                                      (65, 16, (True, False, True)), (300, 5, (True, True, False)),
                                      (97, 128, (False, True, True)), (1100, 16, (True, True, True))],
                         ids=["t1_h16", "t33_h16", "t65_h16", "t300_h5", "t97_h128", "t1100_h16"])
def test_uk_every_launch_gives_the_same_bytes(T, H, mode):
    """Every configuration sums each latent column's 128 products in the same
    order (four 32-wide steps of k, in turn), so the latency configuration
    (one or two 16-column blocks per wavefront, operands from memory) and the
    throughput one (two or four blocks, operands staged in LDS), cached or
    streamed, write identical bytes; the default plan's result also meets
    the bar against the oracle."""
    w = workload(T, H, *mode)
    inp = I.make_uk_inputs(w)
    results = {}
    for name, extra in ALL_LAUNCHES:
        results[name] = run_uk(w, inp, extra, case=f"launch {name}")
    q0, c0 = results["plan"]
    check_all(w, inp, q0, c0)
    for name, (q, c) in results.items():
        assert np.array_equal(q, q0), f"q_out of launch {name} differs from the plan's"
        assert np.array_equal(c, c0), f"cache of launch {name} differs from the plan's"


def test_uk_non_default_stream():
    """The call goes on torch's current stream: launched on a side stream and
    synchronised with that stream alone, it has finished and meets the bar."""
    w = workload(64, 16, True, True, True)
    inp = I.make_uk_inputs(w)
    announce("uk non-default stream")
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q_out = torch.empty(64, 16, I.ROW, dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        M.mla_decode_uk_q_concat_kv_insert(q_out, dev["q_b"][..., :I.UK_K], dev["w_uk_t"], dev["q_b"][..., I.UK_K:],
                                           dev["kv_c"], dev["k_pe"], dev["cache"], dev["slot_mapping"],
                                           dev["positions"], dev["rope_cos_sin"], dev["q_scale"], dev["kv_scale"],
                                           flags_of(w))
    s.synchronize()
    check_all(w, inp, bits(q_out.cpu()), bits(dev["cache"].cpu()))


def test_uk_maximum_token_count_sampled():
    """The largest token count the C ABI accepts at 16 heads (as for the
    epilogue: T * (H + 1) * 72 chunks just below 2^31; one token more is
    refused), in the throughput configuration with streaming stores: about
    31 GB of device buffers drawn on the device.  Tails, cache rows and the
    latent columns of both ends, of the first and last tokens of token ranges
    and of a random sample of tokens are checked against the oracle, and the
    untouched cache rows are still zero."""
    H = 16
    T = (2 ** 31 - 1) // (72 * (H + 1))
    w = workload(T, H, True, True, True)
    flags = flags_of(w)
    d = M.Dims(num_tokens=T, num_heads=H, num_blocks=w.num_blocks, block_size=w.block_size,
               max_position=w.max_position, ql_nope_stride_t=H * 192, ql_nope_stride_h=192,
               q_pe_stride_t=H * 192, q_pe_stride_h=192, kv_c_stride_t=512, k_pe_stride_t=64)
    p = M.uk_plan(d, flags)
    assert p.mapping == 1 and p.streaming == 1 and p.grid_blocks * p.block_threads < 2 ** 32
    d.num_tokens = T + 1
    with pytest.raises(M.MlaDqError):
        M.uk_plan(d, flags)
    if torch.cuda.mem_get_info()[0] < 40 * (1 << 30):
        pytest.skip("needs about 35 GB of free device memory")
    announce(f"uk maximum size T={T} H={H}: drawing inputs on the device")
    dev = I.make_inputs_on_device(w, DEV, seed=37, uk=True)
    q = torch.empty(T, H, I.ROW, dtype=torch.float8_e4m3fn, device=DEV)
    announce(f"uk maximum size T={T} H={H}: kernel ({p.grid_blocks} workgroups, {p.tokens_per_group} tokens per range)")
    M.mla_decode_uk_q_concat_kv_insert(q, dev["q_nope"], dev["w_uk_t"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                       dev["cache"], dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"],
                                       dev["q_scale"], dev["kv_scale"], flags)
    torch.cuda.synchronize()
    tpg = p.tokens_per_group
    gen = torch.Generator().manual_seed(41)
    idx = torch.cat([torch.arange(64), torch.arange(T - 64, T), torch.arange(0, T, tpg * 997),
                     torch.arange(tpg - 1, T, tpg * 1009), torch.randperm(T, generator=gen)[:1024]])
    idx = torch.unique(idx)
    n = idx.numel()
    di = idx.to(DEV)
    slots = dev["slot_mapping"][di]
    want_q = np.zeros((n, H, I.ROW), dtype=np.uint8)
    want_rows = np.zeros((n, 1, I.ROW), dtype=np.uint8)
    oracle.insert(want_q, np.zeros((n, H, I.NOPE), dtype=np.uint16), bits(dev["q_pe"][di]), bits(dev["kv_c"][di]),
                  bits(dev["k_pe"][di]), want_rows, np.arange(n, dtype=np.int64),
                  dev["positions"][di].cpu().numpy(), dev["rope_cos_sin"].cpu().numpy(),
                  w.q_scale, w.kv_scale, True, True, True)
    got = bits(q[di])
    assert_same(got[..., I.NOPE:], want_q[..., I.NOPE:], "q tails (sampled tokens)")
    rows = dev["cache"].view(-1, I.ROW)
    assert_same(bits(rows[slots]), want_rows.reshape(n, I.ROW), "cache rows (sampled tokens)")
    written = torch.zeros(rows.shape[0], dtype=torch.bool, device=DEV)
    written[dev["slot_mapping"]] = True
    assert int(rows[~written].view(torch.uint8).count_nonzero()) == 0
    check_latent(got[..., :I.NOPE], bits(dev["q_nope"][di]), bits(dev["w_uk_t"]), w, "q latent (sampled tokens)")
    del dev, q, rows, written
    torch.cuda.empty_cache()


def test_uk_graph_replays():
    """The fused call captured in a HIP graph: every replay (with eager work
    and a synchronisation between replays) gives the eager call's bytes."""
    w = workload(64, 16, True, True, True)
    inp = I.make_uk_inputs(w)
    q_ref, cache_ref = run_uk(w, inp, case="graph reference")
    announce("uk graph capture t64 h16")
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q_b = dev["q_b"]
    q_out = torch.empty(64, 16, I.ROW, dtype=torch.float8_e4m3fn, device=DEV)
    cache = dev["cache"].clone()
    run = M.PreparedUkInsert(q_out, q_b[..., :I.UK_K], dev["w_uk_t"], q_b[..., I.UK_K:], dev["kv_c"], dev["k_pe"],
                             cache, dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"], dev["q_scale"],
                             dev["kv_scale"], flags_of(w))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(4):
        q_out.view(torch.uint8).fill_(0xFF)
        cache.copy_(dev["cache"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(bits(q_out.cpu()), q_ref, "q (replay)")
        assert_same(bits(cache.cpu()), cache_ref, "cache (replay)")


def _captured(fn):
    """fn warmed up on a side stream, then captured in a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("T,H", [(1, 16), (64, 16), (8, 128), (200, 16)])
@pytest.mark.parametrize("force", ["plan", "small", "large"])
def test_decode_slice_fused_in_a_graph(T, H, force):
    """The decode-step slice with the W_UK product and the epilogue in one
    launch: q_nope and q_pe are views of the q_b projection's [T,H,192]
    output, k_pe a view of the fused-A output, all captured with the
    producers in a HIP graph.  Every replay meets the bar above against the
    oracle on the materialised inputs."""
    announce(f"fused decode slice in a graph T={T} H={H} configuration={force}")
    import bench
    ds = bench.DecodeSlice(T, H, DEV)
    ds.flags |= {"plan": 0, "small": M.FORCE_SMALL_T, "large": M.FORCE_LARGE_T}[force]
    g = _captured(lambda: ds.step(fused=True))
    q_nope, q_pe, kv_c, k_pe = ds.fused_inputs()
    torch.cuda.synchronize()
    assert q_nope.stride() == (H * 192, 192, 1) and q_pe.stride() == (H * 192, 192, 1)
    assert k_pe.stride() == (2112, 1)
    w = I.custom(T, H, num_blocks=max(1, (T + 63) // 64), rope=True, q_fp8=True, kv_fp8=True)
    inp = I.make_inputs(w)
    inp.update(q_nope=q_nope.cpu().contiguous(), q_pe=q_pe.cpu().contiguous(), kv_c=kv_c.cpu().contiguous(),
               k_pe=k_pe.cpu().contiguous(), w_uk_t=ds.w_uk_t.cpu())
    for _ in range(3):
        ds.q_out.view(torch.uint8).fill_(0xFF)
        ds.cache.view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_all(w, inp, bits(ds.q_out.cpu()), bits(ds.cache.cpu()))


def test_decode_step_fused_then_attention_in_a_graph():
    """A decode step with the fused W_UK product + epilogue followed by the
    decode attention, captured in one graph: every replay's queries and cache
    meet the bar above against the oracle, and its attention output is
    bit-identical to an eager attention call on those same queries and cache
    (the attention itself is checked against its oracle elsewhere)."""
    import bench
    B, H, L = 6, 16, 333
    st = bench.DecodeStep(B, H, L, DEV)
    announce(f"fused decode step graph B={B} H={H} L={L}")
    cache0 = st.cache.cpu().clone()       # the synthetic context, before any step writes to it
    g = _captured(lambda: st.step(fused=True))
    q_nope, q_pe, kv_c, k_pe = st.fused_inputs()
    torch.cuda.synchronize()
    w = I.custom(B, H, num_blocks=st.w.num_blocks, rope=True, q_fp8=True, kv_fp8=True)
    inp = dict(q_nope=q_nope.cpu().contiguous(), q_pe=q_pe.cpu().contiguous(), kv_c=kv_c.cpu().contiguous(),
               k_pe=k_pe.cpu().contiguous(), w_uk_t=st.w_uk_t.cpu(), cache=cache0,
               slot_mapping=st.slots.cpu(), positions=st.positions.cpu(), rope_cos_sin=st.table.cpu(),
               q_scale=st.q_scale.cpu(), kv_scale=st.kv_scale.cpu())
    for _ in range(3):
        st.out.view(torch.int16).fill_(-1)
        st.q_out.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_all(w, inp, bits(st.q_out.cpu()), bits(st.cache.cpu()))
        out_graph = st.out.clone()
        st.out.view(torch.int16).fill_(-1)
        st.attn()
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), out_graph.view(torch.int16))
