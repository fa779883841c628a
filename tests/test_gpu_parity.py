"""GPU parity: the gfx950 kernel, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bar: bit-exact for every copied element and every E4M3 code; rotated bf16
outputs within 1e-2 absolute (and, since both sides evaluate the rotation
with the same fp32 operation order, bit-exact as well).  NaN codes are
compared as NaN.  q_out is poison-filled (0xFF) before each call and guard
bands around q_out and the cache catch stray writes; caches start from a
random background where the test is about untouched rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import mla_decode_concat_amd as M
from mla_decode_concat_amd import inputs as I
import oracle
from tests._util import bits, oracle_run

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD_ROWS = 2


def announce(case: str) -> None:
    sys.__stderr__.write(f"[gpu-case] {case}\n")
    sys.__stderr__.flush()


def flags_of(w: I.Workload) -> int:
    f = (M.ROPE if w.rope else 0) | (M.Q_FP8 if w.q_fp8 else 0) | (M.KV_FP8 if w.kv_fp8 else 0)
    if w.dtype == "fp16":
        f |= M.FP16
    if w.rope and w.rope_style == "gptj":
        f |= M.ROPE_GPTJ
    if w.rope and w.table_dtype == "bf16":
        f |= M.TABLE_BF16
    return f


def run_gpu(w: I.Workload, inp: dict, extra_flags: int = 0, cache_init: np.ndarray | None = None,
            views: dict | None = None, case: str = ""):
    """Run the kernel; returns (q bits, cache bits) and checks the guards."""
    announce(f"{case} {w.describe()} flags+{extra_flags:#x}")
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
    elif cache_init.dtype == np.uint16:
        cache_cpu = torch.from_numpy(cache_init.view(np.int16).copy()).view(kvdt)
    else:
        cache_cpu = torch.from_numpy(cache_init.copy()).view(kvdt)
    NB, BS = cache_cpu.shape[0], cache_cpu.shape[1]
    cbig = torch.empty(NB + 2 * GUARD_ROWS, BS, I.ROW, dtype=kvdt, device=DEV)
    gen = torch.Generator().manual_seed(1234)
    guard = torch.randint(0, 256, (GUARD_ROWS, BS, I.ROW * cbig.element_size()), generator=gen,
                          dtype=torch.uint8)
    cbig.view(torch.uint8)[:GUARD_ROWS] = guard.to(DEV)
    cbig.view(torch.uint8)[-GUARD_ROWS:] = guard.to(DEV)
    cache = cbig[GUARD_ROWS:GUARD_ROWS + NB]
    cache.copy_(cache_cpu.to(DEV))
    views = views or {}
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    for k, fn in views.items():
        dev[k] = fn(dev[k])
    M.mla_decode_q_concat_kv_insert(q_out, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                    cache, dev["slot_mapping"], dev["positions"],
                                    dev["rope_cos_sin"], dev["q_scale"], dev["kv_scale"],
                                    flags_of(w) | extra_flags)
    torch.cuda.synchronize()
    qb = qbig.view(torch.uint8).cpu()
    assert torch.all(qb[:pad * qbig.element_size()] == 0xFF), "write before q_out"
    assert torch.all(qb[(pad + n_q) * qbig.element_size():] == 0xFF), "write after q_out"
    cb = cbig.view(torch.uint8).cpu()
    assert torch.equal(cb[:GUARD_ROWS], guard) and torch.equal(cb[-GUARD_ROWS:], guard), \
        "write outside the cache"
    return bits(q_out.cpu()), bits(cache.cpu())


def _nan_mask(x: np.ndarray, fp16: bool = False) -> np.ndarray:
    if x.dtype == np.uint8:
        return (x & 0x7F) == 0x7F
    if fp16:
        return ((x & 0x7C00) == 0x7C00) & ((x & 0x3FF) != 0)
    return ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)


def assert_same(got: np.ndarray, want: np.ndarray, what: str, fp16: bool = False):
    assert got.shape == want.shape and got.dtype == want.dtype, what
    ng, nw = _nan_mask(got, fp16), _nan_mask(want, fp16)
    bad = np.nonzero((ng != nw) | (~nw & (got != want)))
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} mismatches, first at {idx}: "
                             f"got {got[idx]:#x} want {want[idx]:#x}")


def _act_value(x: np.ndarray, fp16: bool) -> np.ndarray:
    if fp16:
        return x.view(np.float16).astype(np.float32)
    return (x.astype(np.uint32) << 16).view(np.float32)


def check_against_oracle(w: I.Workload, inp: dict, q, cache, cache_init=None):
    want_q, want_cache = oracle_run(w, inp, cache_init=cache_init)
    fp16 = w.dtype == "fp16"
    if w.rope and not w.q_fp8:
        # the stated bar on rotated unquantised outputs first
        g, r = _act_value(q[..., 512:], fp16), _act_value(want_q[..., 512:], fp16)
        fin = np.isfinite(r)
        assert np.all(np.abs(g[fin] - r[fin]) <= 1e-2), "rotated q beyond 1e-2"
    assert_same(q, want_q, "q_out", fp16 and not w.q_fp8)
    assert_same(cache, want_cache, "cache", fp16 and not w.kv_fp8)


@pytest.mark.parametrize("name", I.WORKLOAD_ORDER)
def test_workload_matches_oracle(name):
    w = I.WORKLOADS[name]
    inp = I.make_inputs(w)
    q, cache = run_gpu(w, inp, case=f"workload {name}")
    check_against_oracle(w, inp, q, cache)


LAUNCHES = [M.FORCE_SMALL_T | M.FORCE_CACHED, M.FORCE_SMALL_T | M.FORCE_STREAM,
            M.FORCE_MID_T | M.FORCE_CACHED, M.FORCE_MID_T | M.FORCE_STREAM,
            M.FORCE_LARGE_T | M.FORCE_CACHED, M.FORCE_LARGE_T | M.FORCE_STREAM]

VARIANTS = [("fp16", "neox", "f32"), ("bf16", "gptj", "f32"), ("bf16", "neox", "bf16"),
            ("fp16", "gptj", "bf16")]


@pytest.mark.parametrize("name", ["t1_h16_copy", "t64_h16_rope_fp8", "t65_h16_rope_fp8",
                                  "t256_h128_rope_qfp8"])
def test_forced_launches_agree(name):
    """All three mappings and both cache policies give identical bytes on
    identical inputs (the page's split path is bitwise identical to the
    unsplit one)."""
    w = I.WORKLOADS[name]
    inp = I.make_inputs(w)
    outs = [run_gpu(w, inp, f, case=f"launch {f:#x} {name}") for f in LAUNCHES]
    for q, c in outs[1:]:
        assert np.array_equal(q, outs[0][0]) and np.array_equal(c, outs[0][1])
    check_against_oracle(w, inp, *outs[0])


@pytest.mark.parametrize("num_tokens", [64, 65])
def test_page_row_split_boundary(num_tokens):
    """The page's boundary test through the page's call: q == cat(ql_nope,
    q_pe) and the cache rows at the slots == cat(kv_c, k_pe); the rest of the
    zero cache stays zero."""
    announce(f"page boundary T={num_tokens}")
    w = I.custom(num_tokens, 16)
    inp = I.make_inputs(w)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q = M.fused_mla_decode_q_concat_kv_cache_insert(dev["ql_nope"], dev["q_pe"], dev["kv_c"],
                                                    dev["k_pe"], dev["cache"], dev["slot_mapping"])
    torch.cuda.synchronize()
    assert torch.equal(q.cpu(), torch.cat([inp["ql_nope"], inp["q_pe"]], dim=-1))
    rows = dev["cache"].cpu().view(-1, I.ROW)
    slots = inp["slot_mapping"]
    assert torch.equal(rows[slots], torch.cat([inp["kv_c"], inp["k_pe"]], dim=-1))
    mask = torch.ones(rows.shape[0], dtype=torch.bool)
    mask[slots] = False
    assert torch.all(rows[mask].view(torch.int16) == 0)


FLAG_SETS = [(r, q, k) for r in (False, True) for q in (False, True) for k in (False, True)]


@pytest.mark.parametrize("T,H", [(1, 1), (2, 3), (7, 16), (33, 5), (63, 16), (100, 1),
                                 (129, 7), (300, 128), (255, 128), (1000, 16)])
@pytest.mark.parametrize("fl", FLAG_SETS, ids=lambda f: "r%dq%dk%d" % f)
def test_ragged_shapes_all_modes(T, H, fl):
    rope, qf, kf = fl
    if T * (H + 1) > 40000 and fl != (True, True, True):
        pytest.skip("large shape covered in the all-on mode only")
    w = I.custom(T, H, num_blocks=max(1, (T + 63) // 64) + 1, rope=rope, q_fp8=qf, kv_fp8=kf,
                 q_scale=0.04, kv_scale=0.3)
    inp = I.make_inputs(w, seed=T * 131 + H)
    rng = np.random.default_rng(T + H)
    init = rng.integers(0, 256, size=(w.num_blocks, 64, 576 * (1 if kf else 2)), dtype=np.uint8)
    init = init.view(np.uint8 if kf else np.uint16)
    if not kf:
        init = init & np.uint16(0x3FFF)   # finite bf16 background
    q, cache = run_gpu(w, inp, cache_init=init, case=f"ragged T={T} H={H} {fl}")
    check_against_oracle(w, inp, q, cache, cache_init=init)


@pytest.mark.parametrize("T,H", [(1, 1), (31, 1), (32, 1), (33, 1), (97, 1), (250, 2), (77, 3)])
@pytest.mark.parametrize("fl", [f for f in FLAG_SETS if f[0]], ids=lambda f: "r%dq%dk%d" % f)
def test_throughput_mapping_few_heads(T, H, fl):
    """The throughput mapping stages the rope-table rows of the tokens each
    workgroup covers in LDS.  With one head a workgroup's 64 tail rows span
    33 tokens, the most the stage holds; ragged T leaves a partial last
    workgroup.  Forced throughput mapping against the oracle, and equal to
    the latency mapping, with a position table of distinct rows."""
    rope, qf, kf = fl
    w = I.custom(T, H, num_blocks=(T + 63) // 64 + 1, rope=rope, q_fp8=qf, kv_fp8=kf,
                 q_scale=0.04, kv_scale=0.3)
    inp = I.make_inputs(w, seed=7 * T + H)
    ql, cl = run_gpu(w, inp, M.FORCE_LARGE_T, case=f"few heads large T={T} H={H} {fl}")
    qs, cs = run_gpu(w, inp, M.FORCE_SMALL_T, case=f"few heads small T={T} H={H} {fl}")
    qm, cm = run_gpu(w, inp, M.FORCE_MID_T, case=f"few heads mid T={T} H={H} {fl}")
    assert np.array_equal(ql, qs) and np.array_equal(cl, cs)
    assert np.array_equal(qm, qs) and np.array_equal(cm, cs)
    check_against_oracle(w, inp, ql, cl)


@pytest.mark.parametrize("dtype,style,table", [("fp16", "neox", "f32"), ("bf16", "gptj", "bf16"),
                                               ("fp16", "gptj", "bf16"), ("bf16", "neox", "bf16")],
                         ids=lambda v: str(v))
def test_throughput_mapping_few_heads_variants(dtype, style, table):
    """The LDS-staged table rows in the variant layouts (bf16 table rows are
    half as long), one head, ragged T, forced throughput mapping."""
    w = I.custom(95, 1, num_blocks=3, rope=True, q_fp8=False, kv_fp8=True, q_scale=0.04,
                 kv_scale=0.3, dtype=dtype, rope_style=style, table_dtype=table)
    inp = I.make_inputs(w, seed=95)
    ql, cl = run_gpu(w, inp, M.FORCE_LARGE_T, case=f"few heads variant {dtype}/{style}/{table}")
    check_against_oracle(w, inp, ql, cl)


@pytest.mark.parametrize("scale", [1.0, 0.05, 2.0 ** -4, 3.7])
def test_e4m3_exhaustive_all_bf16_inputs(scale):
    """Every bf16 bit pattern through the quantiser, in the latent part, the
    positional part and the cache row (rotation off, then on)."""
    T, H = 8, 16
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    for rope in (False, True):
        w = I.custom(T, H, num_blocks=1, rope=rope, q_fp8=True, kv_fp8=True, q_scale=scale,
                     kv_scale=scale)
        inp = I.make_inputs(w, seed=17)
        inp["ql_nope"] = allbits.view(T, H, 512).clone()
        perm = torch.randperm(65536, generator=torch.Generator().manual_seed(3))
        inp["q_pe"] = allbits[perm[:T * H * 64]].view(T, H, 64).clone()
        inp["kv_c"] = allbits[perm[:T * 512]].view(T, 512).clone()
        inp["k_pe"] = allbits[perm[-T * 64:]].view(T, 64).clone()
        q, cache = run_gpu(w, inp, case=f"e4m3 exhaustive scale={scale} rope={rope}")
        check_against_oracle(w, inp, q, cache)


def test_rotation_on_all_bf16_tails():
    """Every bf16 pattern as a positional element (bf16 output): rounding,
    signed zeros, infinities and NaN through the rotation."""
    T, H = 64, 16
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    w = I.custom(T, H, num_blocks=1, rope=True)
    inp = I.make_inputs(w, seed=21)
    inp["q_pe"] = allbits.view(T, H, 64).clone()
    q, cache = run_gpu(w, inp, case="rope all-bf16 tails")
    want_q, want_cache = oracle_run(w, inp)
    assert_same(q, want_q, "q_out")
    assert_same(cache, want_cache, "cache")


def test_strided_input_views():
    """Inputs as row-strided views of larger buffers."""
    w = I.custom(37, 16, num_blocks=2, rope=True, q_fp8=True, kv_fp8=False)
    inp = I.make_inputs(w, seed=5)
    T, H = w.tokens, w.heads

    def wide(x, extra):  # embed the last dim in a wider row, return the view
        shape = list(x.shape)
        big = torch.zeros(shape[:-1] + [shape[-1] + extra], dtype=x.dtype, device=x.device)
        big[..., 8:8 + shape[-1]] = x
        return big[..., 8:8 + shape[-1]]
    views = {
        "ql_nope": lambda x: wide(x, 64),                         # head stride 576
        "q_pe": lambda x: wide(x.reshape(T, H, 64), 128),         # head stride 192
        "kv_c": lambda x: wide(x, 64),                            # token stride 576
        "k_pe": lambda x: wide(x, 520),                           # token stride 584
    }
    q, cache = run_gpu(w, inp, views=views, case="strided views")
    check_against_oracle(w, inp, q, cache)


SLOT_JUNK = (-1, -7, -(1 << 40), -(1 << 63))
POS_JUNK = (-5, -1, -(1 << 63), (1 << 63) - 1)


def _out_of_range(inp: dict, w: I.Workload, seed: int, frac: float = 0.25):
    """Replace a seeded fraction of the slots by padding or out-of-range
    values (-1, -7, the slot count and past it, +-2^40, int64 extremes) and,
    with rotation, of the positions by values outside [0, max_position)."""
    rng = np.random.default_rng(seed)
    S, T = w.num_slots, w.tokens
    junk = np.array(SLOT_JUNK + (S, S + 5, 1 << 40, (1 << 63) - 1), dtype=np.int64)
    slots = inp["slot_mapping"].numpy().copy()
    pick = rng.random(T) < frac
    slots[pick] = rng.choice(junk, int(pick.sum()))
    inp["slot_mapping"] = torch.from_numpy(slots)
    if w.rope:
        pjunk = np.array(POS_JUNK + (w.max_position, w.max_position + 3, 1 << 40), dtype=np.int64)
        pos = inp["positions"].numpy().copy()
        pick = rng.random(T) < frac
        pos[pick] = rng.choice(pjunk, int(pick.sum()))
        inp["positions"] = torch.from_numpy(pos)
    return inp


def _background(w: I.Workload, seed: int) -> np.ndarray:
    """A random cache background (finite bf16 values, or any E4M3 byte)."""
    rng = np.random.default_rng(seed)
    init = rng.integers(0, 256, size=(w.num_blocks, w.block_size, 576 * (1 if w.kv_fp8 else 2)),
                        dtype=np.uint8)
    if w.kv_fp8:
        return init
    return init.view(np.uint16) & np.uint16(0x3FFF)


# (T, H, max_position): one tail step; a throughput workgroup whose staged
# table rows include clamped positions (1-3 heads, ragged T >= 97); the mid
# and throughput mappings at 16 heads
EDGE_SHAPES = [(6, 4, 16), (97, 1, 16), (130, 2, 77), (200, 3, 4096), (333, 16, 64)]


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda f: f"{f:#x}")
@pytest.mark.parametrize("T,H,maxpos", EDGE_SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("kf", [False, True], ids=["kv", "KV8"])
def test_out_of_range_slots_and_positions(T, H, maxpos, kf, launch):
    """Padding (-1) and out-of-range slots skip the cache row and nothing
    else; out-of-range positions are clamped into the table.  Under every
    mapping and cache policy, on a random cache background."""
    w = I.custom(T, H, num_blocks=(T + 63) // 64 + 1, rope=True, q_fp8=True, kv_fp8=kf,
                 max_position=maxpos, q_scale=0.04, kv_scale=0.3)
    inp = _out_of_range(I.make_inputs(w, seed=4 + T), w, seed=T * 7 + H)
    init = _background(w, seed=T)
    q, cache = run_gpu(w, inp, launch, cache_init=init, case=f"out-of-range T={T} H={H}")
    check_against_oracle(w, inp, q, cache, cache_init=init)


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda f: f"{f:#x}")
def test_out_of_range_slots_without_rotation(launch):
    """The copy path (no positions read) with padding and out-of-range
    slots, under every mapping and cache policy."""
    w = I.custom(150, 2, num_blocks=4, q_scale=0.04, kv_scale=0.3)
    inp = _out_of_range(I.make_inputs(w, seed=8), w, seed=9, frac=0.5)
    init = _background(w, seed=10)
    q, cache = run_gpu(w, inp, launch, cache_init=init, case="out-of-range slots, copy path")
    check_against_oracle(w, inp, q, cache, cache_init=init)


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda f: f"{f:#x}")
@pytest.mark.parametrize("T,H", [(3, 2), (120, 3)])
def test_duplicate_slots_leave_one_candidate(T, H, launch):
    """Tokens that share a slot: every 8-element chunk of that row comes from
    one of them (the header's contract); rows of unique slots are exact."""
    w = I.custom(T, H, num_blocks=(T + 63) // 64 + 1, rope=True, kv_fp8=True, kv_scale=0.3)
    inp = I.make_inputs(w, seed=2 + T)
    slots = inp["slot_mapping"].numpy().copy()
    groups = [[0, 1]] if T == 3 else [[0, 1, 2], [5, 60], [33, 119, 64, 90]]
    for g in groups:
        slots[g] = slots[g[0]]
    inp["slot_mapping"] = torch.from_numpy(slots)
    q, cache = run_gpu(w, inp, launch, case=f"duplicate slots T={T}")
    want_q, want_cache = oracle_run(w, inp)
    assert_same(q, want_q, "q_out")
    rows, want_rows = cache.reshape(-1, 576), want_cache.reshape(-1, 576)
    shared = {int(slots[g[0]]): g for g in groups}
    keep = np.ones(rows.shape[0], dtype=bool)
    keep[list(shared)] = False
    assert_same(rows[keep], want_rows[keep], "cache rows of unique slots and untouched rows")
    w1 = I.custom(1, H, num_blocks=1, rope=True, kv_fp8=True, kv_scale=0.3)
    for s_, g in shared.items():
        cands = []
        for t in g:       # the row token t alone would write
            sub = dict(inp, slot_mapping=torch.tensor([0], dtype=torch.int64),
                       cache=torch.zeros(1, 64, 576, dtype=torch.float8_e4m3fn))
            for k in ("ql_nope", "q_pe", "kv_c", "k_pe", "positions"):
                sub[k] = inp[k][t:t + 1].clone()
            cands.append(oracle_run(w1, sub)[1].reshape(-1, 576)[0].reshape(72, 8))
        got = rows[s_].reshape(72, 8)
        for c in range(72):
            assert any(np.array_equal(got[c], cand[c]) for cand in cands), (s_, c)


def _run_subsets(w: I.Workload, inp: dict, order, launch: int, init: np.ndarray):
    """Calls restricted to row subsets, in the given order, on one poisoned
    q_out and one cache (random background); returns (q bits, cache bits)."""
    qdt = torch.float8_e4m3fn if w.q_fp8 else w.torch_dtype
    kvdt = torch.float8_e4m3fn if w.kv_fp8 else w.torch_dtype
    q_out = torch.empty(w.tokens, w.heads, I.ROW, dtype=qdt, device=DEV)
    q_out.view(torch.uint8).fill_(0xFF)
    src = init.view(np.int16) if init.dtype == np.uint16 else init
    cache = torch.from_numpy(src.copy()).view(kvdt).to(DEV)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    for sub in order:
        announce(f"row subset {sub:#x} {w.describe()} launch {launch:#x}")
        M.mla_decode_q_concat_kv_insert(q_out, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                        cache, dev["slot_mapping"], dev["positions"],
                                        dev["rope_cos_sin"], dev["q_scale"], dev["kv_scale"],
                                        flags_of(w) | sub | launch)
    torch.cuda.synchronize()
    return bits(q_out.cpu()), bits(cache.cpu())


@pytest.mark.parametrize("launch", [0] + LAUNCHES, ids=lambda f: f"{f:#x}")
@pytest.mark.parametrize("T,H", [(1, 16), (64, 16), (97, 1), (300, 3)])
def test_row_subsets_compose(T, H, launch):
    """A call restricted to the query rows writes q_out and leaves the cache
    alone; one restricted to the cache rows writes only the cache rows; the
    two together, in either order, give the oracle's bytes.  Under every
    mapping and cache policy (a cache-rows launch with one head stages one
    table row per tail row in the throughput mapping)."""
    w = I.custom(T, H, num_blocks=(T + 63) // 64 + 1, rope=True, q_fp8=True, kv_fp8=True,
                 q_scale=0.04, kv_scale=0.3)
    inp = _out_of_range(I.make_inputs(w, seed=60 + T), w, seed=61 + H, frac=0.1)
    init = _background(w, seed=62)
    want_q, want_cache = oracle_run(w, inp, cache_init=init)
    q, cache = _run_subsets(w, inp, [M.Q_ROWS_ONLY], launch, init)
    assert_same(q, want_q, "q_out (query rows only)")
    assert np.array_equal(cache, init), "a query-rows launch touched the cache"
    q, cache = _run_subsets(w, inp, [M.CACHE_ROWS_ONLY], launch, init)
    assert np.all(q == (0xFF if w.q_fp8 else 0xFFFF)), "a cache-rows launch touched q_out"
    assert_same(cache, want_cache, "cache (cache rows only)")
    for order in ([M.Q_ROWS_ONLY, M.CACHE_ROWS_ONLY], [M.CACHE_ROWS_ONLY, M.Q_ROWS_ONLY]):
        q, cache = _run_subsets(w, inp, order, launch, init)
        assert_same(q, want_q, "q_out")
        assert_same(cache, want_cache, "cache")


@pytest.mark.parametrize("dtype,style,table", VARIANTS, ids=["-".join(v) for v in VARIANTS])
def test_row_subsets_variants(dtype, style, table):
    w = I.custom(130, 2, num_blocks=4, rope=True, q_fp8=False, kv_fp8=True, q_scale=0.04,
                 kv_scale=0.3, dtype=dtype, rope_style=style, table_dtype=table)
    inp = I.make_inputs(w, seed=63)
    init = _background(w, seed=64)
    want_q, want_cache = oracle_run(w, inp, cache_init=init)
    for launch in (M.FORCE_SMALL_T, M.FORCE_LARGE_T):
        q, cache = _run_subsets(w, inp, [M.CACHE_ROWS_ONLY, M.Q_ROWS_ONLY], launch, init)
        assert_same(q, want_q, "q_out", dtype == "fp16")
        assert_same(cache, want_cache, "cache")


def test_zero_tokens_launches_nothing():
    w = I.custom(0, 16, num_blocks=1)
    inp = I.make_inputs(w)
    q, cache = run_gpu(w, inp, case="T=0")
    assert q.size == 0 and np.all(cache == 0)


def test_non_default_stream():
    announce("non-default stream")
    w = I.WORKLOADS["t64_h16_rope_fp8"]
    inp = I.make_inputs(w)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        q = M.fused_mla_decode_q_concat_kv_cache_insert(
            dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"], dev["cache"],
            dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"], dev["q_scale"],
            dev["kv_scale"], q_fp8=True)
    s.synchronize()
    want_q, want_cache = oracle_run(w, inp)
    assert_same(bits(q.cpu()), want_q, "q_out")
    assert_same(bits(dev["cache"].cpu()), want_cache, "cache")


def test_prepared_insert_matches_oracle_twice():
    announce("prepared insert")
    w = I.WORKLOADS["t65_h16_rope_fp8"]
    inp = I.make_inputs(w)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q = torch.empty(w.tokens, w.heads, 576, dtype=torch.float8_e4m3fn, device=DEV)
    op = M.PreparedInsert(q, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"], dev["cache"],
                          dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"],
                          dev["q_scale"], dev["kv_scale"], flags_of(w))
    want_q, want_cache = oracle_run(w, inp)
    for _ in range(2):
        q.view(torch.uint8).fill_(0xFF)
        op()
        torch.cuda.synchronize()
        assert_same(bits(q.cpu()), want_q, "q_out")
        assert_same(bits(dev["cache"].cpu()), want_cache, "cache")


def test_graph_replays_match_eager():
    """The call captured in a HIP graph, replayed several times with eager
    work in between, gives the eager bytes every time."""
    announce("graph replay")
    w = I.WORKLOADS["t64_h16_rope_fp8"]
    inp = I.make_inputs(w)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q = torch.empty(w.tokens, w.heads, 576, dtype=torch.float8_e4m3fn, device=DEV)
    op = M.PreparedInsert(q, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"], dev["cache"],
                          dev["slot_mapping"], dev["positions"], dev["rope_cos_sin"],
                          dev["q_scale"], dev["kv_scale"], flags_of(w))
    want_q, want_cache = oracle_run(w, inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op()
    for _ in range(3):
        q.view(torch.uint8).fill_(0xFF)
        dev["cache"].view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(bits(q.cpu()), want_q, "q_out")
        assert_same(bits(dev["cache"].cpu()), want_cache, "cache")



@pytest.mark.parametrize("dtype,style,table", VARIANTS, ids=["-".join(v) for v in VARIANTS])
@pytest.mark.parametrize("qf,kf", [(False, False), (True, False), (False, True), (True, True)],
                         ids=["q-kv", "Q8-kv", "q-KV8", "Q8-KV8"])
@pytest.mark.parametrize("T,H", [(37, 5), (300, 16)])
def test_variants_match_oracle(dtype, style, table, qf, kf, T, H):
    """fp16 activations, interleaved rotation and a bf16 table, in every FP8
    mode, on all three mappings (forced) and against the oracle."""
    w = I.custom(T, H, num_blocks=(T + 63) // 64 + 1, rope=True, q_fp8=qf, kv_fp8=kf,
                 q_scale=0.04, kv_scale=0.3, dtype=dtype, rope_style=style, table_dtype=table)
    inp = I.make_inputs(w, seed=T + H)
    qs, cs = run_gpu(w, inp, M.FORCE_SMALL_T, case=f"variant {dtype}/{style}/{table} small")
    ql, cl = run_gpu(w, inp, M.FORCE_LARGE_T | M.FORCE_STREAM, case=f"variant {dtype}/{style}/{table} large")
    qm, cm = run_gpu(w, inp, M.FORCE_MID_T, case=f"variant {dtype}/{style}/{table} mid")
    assert np.array_equal(qs, ql) and np.array_equal(cs, cl)
    assert np.array_equal(qs, qm) and np.array_equal(cs, cm)
    check_against_oracle(w, inp, qs, cs)


def _random_case(i: int):
    """Seeded random shape and mode: tokens, heads, block size, precision of
    each output, activation type, rotation style and table type, slot
    recipe, and which mapping is forced (if any)."""
    rng = np.random.default_rng(1000 + i)
    H = int(rng.choice([1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 64, 128]))
    T = int(rng.integers(1, max(2, min(3000, 60000 // (H + 1)))))
    bs = int(rng.choice([1, 16, 64, 128]))
    rope, qf, kf = bool(rng.integers(2)), bool(rng.integers(2)), bool(rng.integers(2))
    dtype = "fp16" if rng.integers(4) == 0 else "bf16"
    style = "gptj" if rope and rng.integers(3) == 0 else "neox"
    table = "bf16" if rope and rng.integers(3) == 0 else "f32"
    nb = (T + bs - 1) // bs + int(rng.integers(0, 3))
    force = [0, M.FORCE_SMALL_T, M.FORCE_MID_T, M.FORCE_LARGE_T,
             M.FORCE_LARGE_T | M.FORCE_STREAM][int(rng.integers(5))]
    w = I.custom(T, H, num_blocks=nb, block_size=bs, rope=rope, q_fp8=qf, kv_fp8=kf,
                 q_scale=float(rng.choice([0.05, 0.3, 1.0])), kv_scale=float(rng.choice([0.05, 2.0])),
                 dtype=dtype, rope_style=style, table_dtype=table,
                 max_position=int(rng.choice([1, 77, 4096])))
    junk = float(rng.choice([0.0, 0.0, 0.1, 0.5]))     # share of out-of-range slots/positions
    return w, force, int(rng.integers(1 << 30)), junk


@pytest.mark.parametrize("i", range(24))
def test_seeded_random_shapes_and_modes(i):
    """Random shapes, heads, block sizes, flag and variant combinations and
    launch overrides, some cases with padding or out-of-range slots and
    positions, each against the oracle."""
    w, force, seed, junk = _random_case(i)
    inp = I.make_inputs(w, seed=seed)
    if junk:
        inp = _out_of_range(inp, w, seed=seed + 1, frac=junk)
    q, cache = run_gpu(w, inp, force, case=f"random case {i} (seed {seed}, junk {junk})")
    check_against_oracle(w, inp, q, cache)


@pytest.mark.parametrize("T,H", [(1, 16), (65, 16)])
def test_fp16_copy_path(T, H):
    w = I.custom(T, H, dtype="fp16")
    inp = I.make_inputs(w)
    q, cache = run_gpu(w, inp, case=f"fp16 copy T={T}")
    check_against_oracle(w, inp, q, cache)


@pytest.mark.parametrize("scale", [1.0, 0.05, 3.7])
def test_e4m3_exhaustive_all_fp16_inputs(scale):
    T, H = 8, 16
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.float16)
    for rope, style in ((False, "neox"), (True, "neox"), (True, "gptj")):
        w = I.custom(T, H, num_blocks=1, rope=rope, q_fp8=True, kv_fp8=True, q_scale=scale,
                     kv_scale=scale, dtype="fp16", rope_style=style)
        inp = I.make_inputs(w, seed=19)
        inp["ql_nope"] = allbits.view(T, H, 512).clone()
        perm = torch.randperm(65536, generator=torch.Generator().manual_seed(4))
        inp["q_pe"] = allbits[perm[:T * H * 64]].view(T, H, 64).clone()
        inp["kv_c"] = allbits[perm[:T * 512]].view(T, 512).clone()
        inp["k_pe"] = allbits[perm[-T * 64:]].view(T, 64).clone()
        q, cache = run_gpu(w, inp, case=f"fp16 e4m3 exhaustive scale={scale} rope={rope} {style}")
        check_against_oracle(w, inp, q, cache)


@pytest.mark.parametrize("dtype,style", [("bf16", "gptj"), ("fp16", "neox"), ("fp16", "gptj")])
def test_rotation_on_all_tails_variants(dtype, style):
    """Every bit pattern of the activation type as a positional element
    (unquantised output): rounding, signed zeros, infinities, NaN."""
    T, H = 64, 16
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(tdt)
    w = I.custom(T, H, num_blocks=1, rope=True, dtype=dtype, rope_style=style)
    inp = I.make_inputs(w, seed=23)
    inp["q_pe"] = allbits.view(T, H, 64).clone()
    q, cache = run_gpu(w, inp, case=f"rope all tails {dtype} {style}")
    want_q, want_cache = oracle_run(w, inp)
    assert_same(q, want_q, "q_out", dtype == "fp16")
    assert_same(cache, want_cache, "cache", dtype == "fp16")


def test_page_call_with_variants():
    announce("page call fp16 + gptj + bf16 table")
    w = I.custom(33, 16, num_blocks=1, rope=True, q_fp8=True, dtype="fp16", rope_style="gptj",
                 table_dtype="bf16")
    inp = I.make_inputs(w, seed=31)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q = M.fused_mla_decode_q_concat_kv_cache_insert(
        dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"], dev["cache"], dev["slot_mapping"],
        dev["positions"], dev["rope_cos_sin"], dev["q_scale"], None, q_fp8=True, rope_style="gptj")
    torch.cuda.synchronize()
    want_q, want_cache = oracle_run(w, inp)
    assert_same(bits(q.cpu()), want_q, "q_out")
    assert_same(bits(dev["cache"].cpu()), want_cache, "cache", True)


@pytest.mark.parametrize("T,H", [(64, 16), (8, 128), (1, 16)])
@pytest.mark.parametrize("force", ["plan", "small", "mid", "large"])
@pytest.mark.parametrize("fork", [False, True], ids=["one-launch", "forked"])
def test_decode_slice_views_in_a_graph(T, H, force, fork):
    """The epilogue reads its inputs as strided views of upstream outputs
    (q_pe inside [T,H,192], ql_nope as the transposed [H,T,512] product,
    k_pe inside the [T,2112] fused-A output), captured with the producers in
    a HIP graph, under the plan's mapping and each forced one; forked, the
    cache rows run on a second captured stream beside the q_b and W_UK
    products and the query rows after them.  Every replay equals the oracle
    on the materialised inputs."""
    announce(f"decode slice in a graph T={T} H={H} mapping={force} fork={fork}")
    import bench
    ds = bench.DecodeSlice(T, H, DEV)
    ds.flags |= {"plan": 0, "small": M.FORCE_SMALL_T, "mid": M.FORCE_MID_T,
                 "large": M.FORCE_LARGE_T}[force]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ds.step(fork=fork)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ql_nope, q_pe, kv_c, k_pe = ds.producers()
    assert ql_nope.stride() == (512, T * 512, 1) and q_pe.stride() == (H * 192, 192, 1)
    assert k_pe.stride() == (2112, 1)
    w = I.custom(T, H, num_blocks=max(1, (T + 63) // 64), rope=True, q_fp8=True, kv_fp8=True)
    inp = I.make_inputs(w)
    inp.update(ql_nope=ql_nope.cpu().contiguous(), q_pe=q_pe.cpu().contiguous(),
               kv_c=kv_c.cpu().contiguous(), k_pe=k_pe.cpu().contiguous())
    want_q, want_cache = oracle_run(w, inp)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.step(fork=fork)
    for _ in range(3):
        ds.q_out.view(torch.uint8).fill_(0xFF)
        ds.cache.view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(bits(ds.q_out.cpu()), want_q, "q_out")
        assert_same(bits(ds.cache.cpu()), want_cache, "cache")


def test_binding_rejects_wrong_dtypes():
    w = I.WORKLOADS["t1_h16_copy"]
    inp = I.make_inputs(w)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q = torch.empty(1, 16, 576, dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(ValueError):
        M.mla_decode_q_concat_kv_insert(q, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                        dev["cache"], dev["slot_mapping"])
    q16 = torch.empty(1, 16, 576, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        M.mla_decode_q_concat_kv_insert(q16, dev["ql_nope"].float(), dev["q_pe"], dev["kv_c"],
                                        dev["k_pe"], dev["cache"], dev["slot_mapping"])


def test_maximum_token_count_sampled():
    """The largest token count the C ABI accepts at 16 heads: row indices and
    the T * (H + 1) * 72 chunk count sit just below 2^31 (one token more is
    refused).  Full-size call (about 52 GB of device buffers), then both ends
    and a random sample of tokens against the oracle token by token, every
    sampled cache row, and the untouched cache rows still zero."""
    H = 16
    T = (2 ** 31 - 1) // (72 * (H + 1))
    w = I.custom(T, H, rope=True, q_fp8=True, kv_fp8=True)
    flags = flags_of(w)
    d = M.Dims(num_tokens=T, num_heads=H, num_blocks=w.num_blocks, block_size=w.block_size,
               max_position=w.max_position, ql_nope_stride_t=H * 512, ql_nope_stride_h=512,
               q_pe_stride_t=H * 64, q_pe_stride_h=64, kv_c_stride_t=512, k_pe_stride_t=64)
    assert M.plan(d, flags).total_rows == T * (H + 1)
    d.num_tokens = T + 1
    with pytest.raises(M.MlaDqError):
        M.plan(d, flags)
    if torch.cuda.mem_get_info()[0] < 64 * (1 << 30):
        pytest.skip("needs about 60 GB of free device memory")
    announce(f"maximum size T={T} H={H}: drawing inputs on the device")
    dev = I.make_inputs_on_device(w, DEV, seed=29)
    q = torch.empty(T, H, I.ROW, dtype=torch.float8_e4m3fn, device=DEV)
    announce(f"maximum size T={T} H={H}: kernel")
    M.mla_decode_q_concat_kv_insert(q, dev["ql_nope"], dev["q_pe"], dev["kv_c"], dev["k_pe"],
                                    dev["cache"], dev["slot_mapping"], dev["positions"],
                                    dev["rope_cos_sin"], dev["q_scale"], dev["kv_scale"], flags)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(31)
    idx = torch.cat([torch.arange(64), torch.arange(T - 64, T), torch.randperm(T, generator=gen)[:2048]])
    idx = torch.unique(idx)
    n = idx.numel()
    di = idx.to(DEV)
    slots = dev["slot_mapping"][di]
    want_q = np.zeros((n, H, I.ROW), dtype=np.uint8)
    want_rows = np.zeros((n, 1, I.ROW), dtype=np.uint8)
    oracle.insert(want_q, bits(dev["ql_nope"][di]), bits(dev["q_pe"][di]), bits(dev["kv_c"][di]),
                  bits(dev["k_pe"][di]), want_rows, np.arange(n, dtype=np.int64),
                  dev["positions"][di].cpu().numpy(), dev["rope_cos_sin"].cpu().numpy(),
                  w.q_scale, w.kv_scale, True, True, True)
    assert_same(bits(q[di]), want_q, "q_out (sampled tokens)")
    rows = dev["cache"].view(-1, I.ROW)
    assert_same(bits(rows[slots]), want_rows.reshape(n, I.ROW), "cache rows (sampled tokens)")
    written = torch.zeros(rows.shape[0], dtype=torch.bool, device=DEV)
    written[dev["slot_mapping"]] = True
    assert int(rows[~written].view(torch.uint8).count_nonzero()) == 0
    del dev, q, rows, written
    torch.cuda.empty_cache()
