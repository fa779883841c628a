"""GPU parity of MLA decode attention (include/mla_attn.h): the gfx950
kernels, called through the C ABI, against the float64 oracle
(oracle/attention.py) on the same seeded inputs.

Tolerance, from the kernel's arithmetic, per output element (b, h, d).
Scores are exact bf16 products summed in fp32 (E4M3 operands convert to
bf16 exactly): at 576 terms their error moves each softmax weight by a
relative ~1e-6, far below the next term.  The value product uses the
weights rounded to bf16 (round to nearest even), p_j (1 + d_j) with
|d_j| <= 2^-9, while the normaliser sums the unrounded fp32 weights, so the
output errs by at most 2^-9 sum_j p_j |v_j,d| (p the exact softmax weights).
The fp32 sums over keys, the range merges and the final division add
relative errors of ~1e-5 of the same quantities, and the bf16 output adds at
most 2^-9 |out|.  The test allows twice the two main terms:

    |gpu - ref| <= 2^-8 (sum_j p_j |v_j,d| + |ref|)

with both sums from the float64 oracle.  The output buffer is poisoned with
NaN first, so every element must be written.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import mla_decode_concat_amd as M
from mla_decode_concat_amd import inputs as I
from oracle import attention as A
from tests._util import bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(case: str) -> None:
    sys.__stderr__.write(f"[gpu-case] {case}\n")
    sys.__stderr__.flush()


def oracle_out(w: I.AttnWorkload, inp: dict, seq_lens=None, block_table=None):
    """The float64 oracle's output and the elementwise tolerance
    2^-8 (sum_j p_j |v_j,d| + |ref|)."""
    lens = inp["seq_lens"].numpy() if seq_lens is None else np.asarray(seq_lens)
    table = inp["block_table"].numpy() if block_table is None else np.asarray(block_table)
    ref, mag = A.mla_decode_attention(bits(inp["q"]), bits(inp["cache"]), table, lens, w.sm_scale,
                                      q_scale=w.q_scale if w.q_fp8 else None,
                                      kv_scale=w.kv_scale if w.kv_fp8 else None, with_abs=True)
    return ref, tolerance(ref, mag)


def tolerance(ref: np.ndarray, mag: np.ndarray) -> np.ndarray:
    return 2.0 ** -8 * (mag + np.abs(ref))


def to_device(inp: dict) -> dict:
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_gpu(w: I.AttnWorkload, inp: dict, case: str, max_seq_len=None, stream=None,
            seq_lens=None, block_table=None) -> np.ndarray:
    d = to_device(inp)
    if seq_lens is not None:
        d["seq_lens"] = torch.as_tensor(np.asarray(seq_lens), dtype=torch.int32).to(DEV)
    if block_table is not None:
        d["block_table"] = torch.as_tensor(np.asarray(block_table), dtype=torch.int32).to(DEV)
    out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(-1)                       # 0xFFFF: a bf16 NaN
    prep = M.PreparedAttention(out, d["q"], d["cache"], d["block_table"], d["seq_lens"],
                               w.sm_scale, d["q_scale"], d["kv_scale"], max_seq_len=max_seq_len)
    announce(f"{case} {w.describe()} splits={prep.plan.splits} kps={prep.plan.keys_per_split} "
             f"wgs={prep.plan.workgroups} combine={prep.plan.combine}")
    prep(stream)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol, case):
    assert np.isfinite(got).all(), f"{case}: unwritten or non-finite outputs"
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{case}: {bad.sum()} elements outside the bound; first {idx.tolist()}"
                             f" got {got[bad][:5]} ref {ref[bad][:5]} tol {tol[bad][:5]}")
    rel = err.max() / max(np.abs(ref).max(), 1e-30)
    sys.__stderr__.write(f"[gpu-case] {case}: max |err| {err.max():.3g} (max/ref {rel:.3g})\n")


def check(w: I.AttnWorkload, case: str, seed: int = I.DEFAULT_SEED, **kw):
    inp = I.make_attn_inputs(w, seed)
    got = run_gpu(w, inp, case, **kw)
    seq_lens = kw.get("seq_lens")
    block_table = kw.get("block_table")
    ref_lens = None
    if seq_lens is not None:
        cap = kw.get("max_seq_len") or w.max_blocks * w.block_size
        ref_lens = np.clip(np.asarray(seq_lens), 0, cap)
    ref_table = None
    if block_table is not None:
        ref_table = np.clip(np.asarray(block_table), 0, w.num_blocks - 1)
    ref, tol = oracle_out(w, inp, ref_lens, ref_table)
    assert_close(got, ref, tol, case)
    return got, ref


@pytest.mark.parametrize("name", list(I.ATTN_WORKLOADS))
def test_workloads(name):
    """Each workload at full size in the launch configuration the benchmark
    times.  Up to 64 sequences every output is compared; above that the full
    batch runs and 32 sequences (the first, the last and a seeded sample) are
    compared with the oracle, which computes each sequence on its own."""
    w = I.ATTN_WORKLOADS[name]
    if w.batch <= 64:
        check(w, name)
        return
    inp = I.make_attn_inputs(w)
    got = run_gpu(w, inp, name)
    rng = np.random.default_rng(17)
    idx = np.unique(np.r_[0, w.batch - 1, rng.choice(np.arange(1, w.batch - 1), 30, replace=False)])
    sub = dict(inp, q=inp["q"][idx], block_table=inp["block_table"][idx], seq_lens=inp["seq_lens"][idx])
    ws = dataclasses.replace(w, batch=len(idx), seq_lens=tuple(w.seq_lens[i] for i in idx))
    ref, tol = oracle_out(ws, sub)
    assert_close(got[idx], ref, tol, f"{name} ({len(idx)} sampled sequences)")


RAGGED = (0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1000, 4096)


@pytest.mark.parametrize("q_fp8,kv_fp8", [(False, False), (False, True), (True, False), (True, True)])
def test_ragged_lengths_all_modes(q_fp8, kv_fp8):
    w = I.attn_custom(len(RAGGED), 16, RAGGED, q_fp8=q_fp8, kv_fp8=kv_fp8, name="ragged")
    check(w, f"ragged q_fp8={q_fp8} kv_fp8={kv_fp8}")


@pytest.mark.parametrize("heads", [1, 20, 128])
def test_head_counts(heads):
    w = I.attn_custom(6, heads, (5, 64, 200, 1, 700, 0), kv_fp8=True, name=f"h{heads}")
    check(w, f"heads={heads}")


@pytest.mark.parametrize("block_size", [1, 5, 16, 128])
def test_block_sizes(block_size):
    w = I.attn_custom(4, 16, (3, 130, 517, 64), block_size=block_size, kv_fp8=True,
                      name=f"bs{block_size}")
    check(w, f"block_size={block_size}")


@pytest.mark.parametrize("kv_fp8", [False, True])
@pytest.mark.parametrize("lengths,splits", [((8192, 3000), 128), ((4096, 3000), 64), ((1024,), 16),
                                            ((768, 40, 0), 12), ((700,) * 40, 6)],
                         ids=["128", "64", "16", "12", "6"])
def test_range_merge_group_sizes(lengths, splits, kv_fp8):
    """Few sequences split into many ranges: 128 and 64 ranges (four
    wavefronts share a head's ranges and meet in LDS), 16 and 12 ranges (one
    wavefront takes them in one group of 16), 6 ranges (a group of 8); short
    and empty sequences leave whole ranges without keys."""
    w = I.attn_custom(len(lengths), 16, lengths, kv_fp8=kv_fp8, name=f"ranges{len(lengths)}")
    plan = M.attn_plan(M.AttnDims(w.batch, w.heads, w.num_blocks, w.block_size, w.max_blocks,
                                  w.max_blocks * w.block_size), M.ATTN_KV_FP8 if kv_fp8 else 0)
    assert plan.splits == splits
    check(w, f"ranges lengths={lengths[:3]} kv_fp8={kv_fp8} splits={plan.splits}")


@pytest.mark.parametrize("lengths,kv_fp8", [((1 << 18,), True), ((1 << 18, 3), False)])
def test_long_sequence_many_ranges(lengths, kv_fp8):
    """A sequence of 2^18 cached tokens (4096 pages; 151 or 302 MB of cache):
    256 ranges of 1024 keys, merged by the wide combine kernel in groups of
    16 per wavefront; and, with a bf16 cache, beside it a 3-token sequence
    whose ranges are all but one empty (128 ranges of 2048 keys)."""
    w = I.attn_custom(len(lengths), 16, lengths, kv_fp8=kv_fp8, name="long")
    plan = M.attn_plan(M.AttnDims(w.batch, w.heads, w.num_blocks, w.block_size, w.max_blocks,
                                  w.max_blocks * w.block_size), M.ATTN_KV_FP8 if kv_fp8 else 0)
    assert (plan.splits, plan.keys_per_split) == (256 // len(lengths), 1024 * len(lengths))
    check(w, f"long lengths={lengths} kv_fp8={kv_fp8} splits={plan.splits}", seed=77)


def _random_shape(case: int):
    """A seeded random (batch, heads, lengths, block size, precisions) case:
    lengths mix empty, sub-tile, page-crossing and multi-range sequences."""
    r = np.random.default_rng(1000 + case)
    batch = int(r.integers(1, 7))
    heads = int(r.choice([1, 3, 16, 20, 33]))
    block_size = int(r.choice([1, 7, 16, 64, 96]))
    lengths = tuple(int(x) for x in r.choice([0, 1, 5, 16, 17, 63, 64, 65, 130, 257, 700, 1500], batch))
    q_fp8, kv_fp8 = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    return batch, heads, lengths, block_size, q_fp8, kv_fp8


@pytest.mark.parametrize("case", range(16))
def test_random_shapes(case):
    batch, heads, lengths, block_size, q_fp8, kv_fp8 = _random_shape(case)
    w = I.attn_custom(batch, heads, lengths, block_size=block_size, q_fp8=q_fp8, kv_fp8=kv_fp8,
                      name=f"random{case}")
    check(w, f"random case {case}: B={batch} H={heads} bs={block_size} L={lengths} "
             f"q_fp8={q_fp8} kv_fp8={kv_fp8}", seed=50 + case)


def test_single_range_writes_output_directly():
    """Enough (sequence, head tile) pairs that each sequence is one range:
    the partial kernel normalises and writes bf16 itself (no combine)."""
    w = I.attn_custom(32, 256, tuple(range(1, 320, 10)), kv_fp8=True, name="direct")
    inp = I.make_attn_inputs(w)
    d = to_device(inp)
    out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device=DEV)
    prep = M.PreparedAttention(out, d["q"], d["cache"], d["block_table"], d["seq_lens"],
                               w.sm_scale, d["q_scale"], d["kv_scale"])
    assert prep.plan.splits == 1 and prep.plan.combine == 0
    check(w, "direct")


def test_short_sequences_single_step():
    w = I.attn_custom(9, 16, (1, 2, 3, 8, 16, 31, 33, 63, 64), name="short")
    check(w, "short")


@pytest.mark.parametrize("batch,heads,lengths,q_fp8", [
    (300, 16, tuple((7 * i) % 65 for i in range(300)), True),      # one range per sequence: bf16 written directly
    (1, 16, (1000,), False),                                       # 16 ranges, cached partial results
    (8, 128, (256, 255, 200, 129, 64, 63, 1, 0), False),           # 4 ranges, streamed partial results
], ids=["direct", "split", "split_streamed"])
def test_short_range_kernel(batch, heads, lengths, q_fp8):
    """Plans whose E4M3 ranges hold 64 keys (one tile per compute wavefront)
    run the kernel without loader wavefronts; all three of its forms against
    the oracle, ragged lengths included."""
    w = I.attn_custom(batch, heads, lengths, q_fp8=q_fp8, kv_fp8=True, name="short_range")
    inp = I.make_attn_inputs(w)
    d = to_device(inp)
    out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device=DEV)
    prep = M.PreparedAttention(out, d["q"], d["cache"], d["block_table"], d["seq_lens"],
                               w.sm_scale, d["q_scale"], d["kv_scale"])
    assert prep.plan.keys_per_split == 64 and prep.plan.block_threads == 256
    # partial results stream past the caches from 4 MiB per call
    streamed = bool(prep.plan.combine) and batch * heads * prep.plan.splits * 512 * 4 >= (4 << 20)
    want = {300: (0, False), 1: (1, False), 8: (1, True)}[batch]
    assert (prep.plan.combine, streamed) == want
    check(w, f"short-range kernel B={batch} H={heads}")


def test_all_empty_sequences_give_zeros():
    w = I.attn_custom(3, 16, (0, 0, 0), name="empty")
    inp = I.make_attn_inputs(w)
    got = run_gpu(w, inp, "empty", max_seq_len=0)
    assert (got == 0).all()
    got = run_gpu(w, inp, "empty-capacity")
    assert (got == 0).all()


def test_lengths_are_clamped():
    """Negative lengths count as 0; lengths past max_seq_len count as
    max_seq_len (the header's contract)."""
    w = I.attn_custom(4, 16, (64, 64, 64, 64), name="clamp")
    check(w, "clamp", seq_lens=[-5, 70, 10 ** 6, 33])


def test_explicit_max_seq_len_changes_the_split():
    w = I.attn_custom(2, 16, (900, 1000), kv_fp8=True, name="maxlen")
    got_a, ref = check(w, "maxlen-capacity")
    got_b, _ = check(w, "maxlen-1000", max_seq_len=1000)
    assert np.array_equal(np.isfinite(got_a), np.isfinite(got_b))


def test_out_of_range_pages_are_clamped():
    w = I.attn_custom(2, 16, (200, 130), name="pages")
    inp = I.make_attn_inputs(w)
    table = inp["block_table"].numpy().copy()
    table[0, 1] = -7
    table[1, 2] = w.num_blocks + 100
    check(w, "pages", block_table=table)


def test_side_stream_and_repeat_are_identical():
    w = I.attn_custom(5, 16, (100, 2000, 3, 4096, 65), kv_fp8=True, name="stream")
    inp = I.make_attn_inputs(w)
    a = run_gpu(w, inp, "default-stream")
    s = torch.cuda.Stream()
    b = run_gpu(w, inp, "side-stream", stream=s)
    assert np.array_equal(a, b)


def test_seeds():
    for seed in (1, 2):
        w = I.attn_custom(3, 16, (333, 64, 1500), q_fp8=True, kv_fp8=True, name=f"seed{seed}")
        check(w, f"seed={seed}", seed=seed)


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_nan_in_unused_cache_slots_is_ignored(kv_fp8):
    """Slots past a sequence's length (the tail of its last page, other
    pages) hold NaN; no output may see them."""
    w = I.attn_custom(4, 16, (70, 1, 129, 3000), kv_fp8=kv_fp8, name="nan-slots")
    inp = I.make_attn_inputs(w)
    cache = inp["cache"]
    raw = cache.view(torch.uint8) if kv_fp8 else cache.view(torch.int16)
    used = torch.zeros(w.num_blocks, w.block_size, dtype=torch.bool)
    for b, L in enumerate(w.seq_lens):
        j = torch.arange(L)
        used[inp["block_table"][b, (j // w.block_size).long()].long(), j % w.block_size] = True
    raw[~used] = 0x7F if kv_fp8 else 0x7FC0
    got = run_gpu(w, inp, f"nan-slots kv_fp8={kv_fp8}")
    ref, tol = oracle_out(w, inp)
    assert_close(got, ref, tol, "nan-slots")


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_table_entries_past_the_length_are_ignored(kv_fp8):
    """Block-table entries past each sequence's length hold garbage (negative
    and huge page numbers) and every unused cache slot holds NaN: the
    header allows the kernel to read them, but they may not reach the
    output."""
    w = I.attn_custom(5, 16, (70, 1, 129, 0, 900), kv_fp8=kv_fp8, name="table-garbage")
    inp = I.make_attn_inputs(w)
    cache = inp["cache"]
    raw = cache.view(torch.uint8) if kv_fp8 else cache.view(torch.int16)
    used = torch.zeros(w.num_blocks, w.block_size, dtype=torch.bool)
    table = inp["block_table"].clone()
    g = torch.Generator().manual_seed(11)
    for b, L in enumerate(w.seq_lens):
        j = torch.arange(L)
        used[table[b, (j // w.block_size).long()].long(), j % w.block_size] = True
        n_used = (L + w.block_size - 1) // w.block_size
        tail = table.shape[1] - n_used
        if tail > 0:
            junk = torch.randint(-(2 ** 31), 2 ** 31 - 1, (tail,), generator=g, dtype=torch.int64)
            table[b, n_used:] = junk.to(torch.int32)
    raw[~used] = 0x7F if kv_fp8 else 0x7FC0
    inp["block_table"] = table
    got = run_gpu(w, inp, f"table-garbage kv_fp8={kv_fp8}")
    ref, tol = oracle_out(w, inp)
    assert_close(got, ref, tol, "table-garbage")


@pytest.mark.parametrize("q_fp8", [False, True])
def test_every_e4m3_code_reaches_the_output_exactly(q_fp8):
    """With one key per sequence the softmax weight is exactly 1 and the
    output is that key's value part, rounded to bf16.  With scale 1 every
    finite E4M3 code (all 254) is a bf16 value, so the output must equal
    its decoded value bit for bit: the kernel's E4M3 -> bf16 conversion is
    exact for every code, including subnormals and +-448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    n = len(codes)                                   # 254
    B = (n + 511) // 512 * 2                         # 2 sequences of one key
    w = I.attn_custom(B, 16, 1, q_fp8=q_fp8, kv_fp8=True, kv_scale=1.0, q_scale=1.0,
                      name="codes")
    inp = I.make_attn_inputs(w)
    raw = inp["cache"].view(torch.uint8)
    vals = np.resize(codes, 2 * 512)
    for b in range(B):
        page = int(inp["block_table"][b, 0])
        raw[page, 0, :512] = torch.from_numpy(vals[512 * b:512 * (b + 1)].copy()) if b < 2 \
            else raw[page, 0, :512]
    got = run_gpu(w, inp, f"e4m3 codes q_fp8={q_fp8}")
    for b in range(min(B, 2)):
        want = A.e4m3_decode(vals[512 * b:512 * (b + 1)])
        for h in range(16):
            assert np.array_equal(got[b, h], want), (b, h)


@pytest.mark.parametrize("fork", [False, True], ids=["one-launch", "forked"])
def test_decode_step_graph_epilogue_then_attention(fork):
    """One decode step captured in a HIP graph: the q-path GEMMs, the
    epilogue (writes each sequence's new E4M3 cache row and E4M3 queries),
    then the attention over all L rows.  Every replay equals the epilogue
    oracle followed by the attention oracle (within the attention bound)."""
    import bench
    import oracle
    from tests._util import oracle_run
    B, H, L = 6, 16, 333
    st = bench.DecodeStep(B, H, L, DEV)
    announce(f"decode step graph B={B} H={H} L={L} fork={fork}")
    cache0 = st.cache.cpu().clone()       # the synthetic context, before any step writes to it
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step(fork=fork)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the epilogue's inputs, materialised, and the oracle's epilogue
    ql_nope, q_pe, kv_c, k_pe = st.producers()
    ew = I.custom(B, H, num_blocks=st.w.num_blocks, rope=True, q_fp8=True, kv_fp8=True)
    einp = dict(ql_nope=ql_nope.cpu().contiguous(), q_pe=q_pe.cpu().contiguous(),
                kv_c=kv_c.cpu().contiguous(), k_pe=k_pe.cpu().contiguous(),
                cache=cache0, slot_mapping=st.slots.cpu(), positions=st.positions.cpu(),
                rope_cos_sin=st.table.cpu(), q_scale=st.q_scale.cpu(), kv_scale=st.kv_scale.cpu())
    want_q, want_cache = oracle_run(ew, einp)
    ainp = dict(q=torch.from_numpy(want_q).view(torch.float8_e4m3fn),
                cache=torch.from_numpy(want_cache).view(torch.float8_e4m3fn),
                block_table=st.block_table.cpu(), seq_lens=st.seq_lens.cpu())
    ref, tol = oracle_out(st.w, ainp)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step(fork=fork)
    for _ in range(3):
        st.out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(st.q_out.cpu()), want_q)
        assert np.array_equal(bits(st.cache.cpu()), want_cache)
        assert_close(st.out.float().cpu().numpy().astype(np.float64), ref, tol, "decode step")


def test_workspace_reuse_across_calls_and_shapes():
    """One workspace serves repeated calls and a different problem (it is
    scratch between calls): every result is the same as the first and
    matches the oracle."""
    w1 = I.attn_custom(5, 16, (100, 2000, 3, 4096, 65), kv_fp8=True, name="ws1")
    w2 = I.attn_custom(3, 20, (700, 10, 1500), q_fp8=True, kv_fp8=True, name="ws2")
    d1, d2 = to_device(I.make_attn_inputs(w1)), to_device(I.make_attn_inputs(w2))
    o1 = torch.empty(w1.batch, w1.heads, 512, dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty(w2.batch, w2.heads, 512, dtype=torch.bfloat16, device=DEV)
    sizes = []
    for w, d in ((w1, d1), (w2, d2)):
        dims = M.AttnDims()
        dims.batch, dims.num_heads = w.batch, w.heads
        dims.num_blocks, dims.block_size = w.num_blocks, w.block_size
        dims.max_blocks_per_seq = w.max_blocks
        dims.max_seq_len = w.max_blocks * w.block_size
        sizes.append(M.attn_workspace_size(dims, (M.ATTN_Q_FP8 if w.q_fp8 else 0) | M.ATTN_KV_FP8))
    assert min(sizes) > 0
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=DEV)
    p1 = M.PreparedAttention(o1, d1["q"], d1["cache"], d1["block_table"], d1["seq_lens"],
                             w1.sm_scale, d1["q_scale"], d1["kv_scale"], workspace=ws)
    p2 = M.PreparedAttention(o2, d2["q"], d2["cache"], d2["block_table"], d2["seq_lens"],
                             w2.sm_scale, d2["q_scale"], d2["kv_scale"], workspace=ws)
    announce("workspace reuse")
    p1()
    torch.cuda.synchronize()
    first = o1.clone()
    for _ in range(2):
        o1.view(torch.int16).fill_(-1)
        p1()
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), first.view(torch.int16))
    p2()
    torch.cuda.synchronize()
    inp2 = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d2.items()}
    ref2, tol2 = oracle_out(w2, inp2)
    assert_close(o2.float().cpu().numpy().astype(np.float64), ref2, tol2, "ws2")
    o1.view(torch.int16).fill_(-1)
    p1()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), first.view(torch.int16))
    inp1 = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d1.items()}
    ref1, tol1 = oracle_out(w1, inp1)
    assert_close(first.float().cpu().numpy().astype(np.float64), ref1, tol1, "ws1")
