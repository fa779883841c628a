#!/usr/bin/env python3
"""Benchmark of the fused MLA decode epilogue on one MI355X.

One step = one call of the epilogue (the whole path: index decode, loads,
rotation, quantisation, q write and cache scatter) over one batch of
synthetic input already resident in HBM.  The headline line is the
8192-token prefill-sized workload (H=16, rotation on, bf16 q, e4m3 cache)
as achieved HBM GB/s against the 8 TB/s peak, with the micro-second cost per
call at 1, 64 and 65 tokens beside it.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line on stdout.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_decode_concat_amd as M  # noqa: E402
from mla_decode_concat_amd import inputs as I  # noqa: E402

METRIC = "µs/call at 1/64/65 tokens + achieved HBM GB/s (% of peak) at 8192 tokens"
HEADLINE = "t8192_h16_rope_kvfp8"
LATENCY = ["t1_h16_copy", "t64_h16_rope_fp8", "t65_h16_rope_fp8"]
MID = ["t256_h128_rope_qfp8"]
# The headline shape in the other element type, rotation style and table type.
VARIANTS = {"fp16": dict(dtype="fp16"), "gptj": dict(rope_style="gptj"),
            "table_bf16": dict(table_dtype="bf16"),
            "fp16_gptj_table_bf16": dict(dtype="fp16", rope_style="gptj", table_dtype="bf16")}
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "mla_decode_concat_amd", "csrc", f)
                  for f in ("mla_dq_kernel.hip", "mla_dq_rows.h", "mla_dq_api.hip", "mla_dq_internal.h",
                            "fastdiv.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mla_dq_epilogue_t8192_h16_traffic.json")
ATTN_SOURCES = [os.path.join(ROOT, "mla_decode_concat_amd", "csrc", "mla_attn.hip"),
                os.path.join(ROOT, "include", "mla_attn.h")]
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mla_attn_decode_traffic.json")


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def algorithmic_bytes(w: I.Workload) -> int:
    """Bytes the method must move per call: every input row read once (1152 B
    of bf16 per 576-wide row), every output row written once (576 x 1 or 2
    bytes), the slot (8 B) per token and, with rotation, the position (8 B)
    and one 256-B cos/sin table row per token."""
    T, H = w.tokens, w.heads
    table_row = 128 if w.table_dtype == "bf16" else 256
    read = T * (H * 1152 + 1152 + 8 + (8 + table_row if w.rope else 0))
    write = T * 576 * (H * (1 if w.q_fp8 else 2) + (1 if w.kv_fp8 else 2))
    return read + write


def flags_of(w: I.Workload) -> int:
    f = (M.ROPE if w.rope else 0) | (M.Q_FP8 if w.q_fp8 else 0) | (M.KV_FP8 if w.kv_fp8 else 0)
    if w.dtype == "fp16":
        f |= M.FP16
    if w.rope and w.rope_style == "gptj":
        f |= M.ROPE_GPTJ
    if w.rope and w.table_dtype == "bf16":
        f |= M.TABLE_BF16
    return f


class DeviceSet:
    """One batch of device-resident inputs and outputs for a workload."""

    def __init__(self, w: I.Workload, host: dict, dev: str):
        self.w = w
        self.t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in host.items()}
        self.q = torch.empty(w.tokens, w.heads, I.ROW, device=dev,
                             dtype=torch.float8_e4m3fn if w.q_fp8 else w.torch_dtype)
        self.flags = flags_of(w)
        t = self.t
        self.prepared = M.PreparedInsert(self.q, t["ql_nope"], t["q_pe"], t["kv_c"], t["k_pe"],
                                         t["cache"], t["slot_mapping"], t["positions"],
                                         t["rope_cos_sin"], t["q_scale"], t["kv_scale"],
                                         self.flags)

    def call(self):
        t = self.t
        M.mla_decode_q_concat_kv_insert(self.q, t["ql_nope"], t["q_pe"], t["kv_c"], t["k_pe"],
                                        t["cache"], t["slot_mapping"], t["positions"],
                                        t["rope_cos_sin"], t["q_scale"], t["kv_scale"], self.flags)


def settle(fns: list, ms: float = 40.0) -> None:
    """Untimed back-to-back calls for about `ms` milliseconds before a timed
    measurement.  After the GPU has idled, the first 15-20 ms of sustained
    load run 10-25 % slower than the steady state (measured on the
    256-sequence attention with the shader clock and board power sampled
    every 5 ms: the transient passes while the shader clock steps down from
    2.4 GHz and board power climbs to its limit), so a short timed run
    straight after idle would measure that transient, not the kernel."""
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < ms * 1e-3:
        for _ in range(8):
            fns[i % len(fns)]()
            i += 1
        torch.cuda.synchronize()


def time_calls(sets: list, steps: int, warmup: int) -> dict:
    """Back-to-back calls on torch's current stream (the stream the kernel is
    launched on), bracketed by synchronisation: the host clock gives the wall
    time per call over all `steps`.  HIP events give the average per-launch
    time over calls 2..steps: the start event follows the first call in
    stream order, so the GPU's wait for the host to enqueue that first call
    after the synchronisation (several µs, which 20 steps would spread as
    0.3-0.5 µs over each) is not counted as kernel time."""
    for i in range(warmup):
        sets[i % len(sets)].call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    first = 1 if steps >= 2 else 0
    if first:
        sets[0].call()
    e0.record(stream)
    for i in range(first, steps):
        sets[i % len(sets)].call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"event_ms_per_call": e0.elapsed_time(e1) / (steps - first), "wall_ms_per_call": wall * 1e3 / steps}


def time_graph(sets: list, calls: int = 100, replays: int = 20) -> float:
    """Device µs per call when `calls` launches (cycling through the sets) are
    captured in one HIP graph and replayed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            s.prepared()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            sets[i % len(sets)].prepared()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (calls * replays)


def time_queued(s, calls: int = 200) -> float:
    """Device µs per call for launches queued behind a spin kernel, so that
    the host has enqueued them all before the first one starts."""
    for _ in range(10):
        s.prepared()
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        s.prepared()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def time_host(fn, calls: int = 2000) -> float:
    """Host µs per call of a Python-level launch path (GPU work drained once
    at the end)."""
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return (t1 - t0) * 1e6 / calls


class DecodeSlice:
    """One GPU's share (H heads) of the MLA path around the epilogue, with
    random weights.  The fused-A projection [T,7168] x [7168, 1536+576] gives
    q_a and kv_a.  q_a goes through its RMSNorm, the q_b projection
    [T,1536] x [1536, H*192] and the per-head W_UK product [H,T,128] x
    [H,128,512], which give ql_nope and q_pe; the first 512 elements of kv_a
    go through their RMSNorm (kv_c), the last 64 are k_pe.  The epilogue reads
    ql_nope, q_pe and k_pe as strided views of those outputs (no copies), or,
    for comparison, from contiguous copies.

    With ``fork`` the epilogue runs as two launches: the cache rows (which
    need only kv_c and k_pe) on a second stream right after the kv norm,
    beside the q_b and W_UK products, and the query rows after W_UK; the
    main stream then waits for both.

    With ``fused`` the W_UK product and the epilogue are one launch
    (mla_decode_uk_q_concat_kv_insert): it reads q_nope and q_pe as views of
    the q_b output and W_UK transposed once ([H,512,128]); ql_nope is never
    stored."""

    def __init__(self, T: int, H: int, dev: str, seed: int = 3):
        g = torch.Generator(device="cpu").manual_seed(seed)

        def rnd(*shape, scale=1.0):
            return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).to(dev)
        self.T, self.H = T, H
        self.hidden = rnd(T, 7168)
        self.w_a = rnd(7168, 1536 + 576, scale=7168 ** -0.5)
        self.w_qb = rnd(1536, H * 192, scale=1536 ** -0.5)
        self.w_uk = rnd(H, 128, 512, scale=128 ** -0.5)
        self.w_uk_t = self.w_uk.transpose(1, 2).contiguous()      # [H, 512, 128], done once
        self.g_q = rnd(1536, scale=0.1) + 1.0
        self.g_kv = rnd(512, scale=0.1) + 1.0
        w = I.custom(T, H, num_blocks=max(1, (T + 63) // 64), rope=True, q_fp8=True, kv_fp8=True)
        host = I.make_inputs(w)
        self.cache = host["cache"].to(dev)
        self.slots = host["slot_mapping"].to(dev)
        self.positions = host["positions"].to(dev)
        self.table = host["rope_cos_sin"].to(dev)
        self.q_scale = host["q_scale"].to(dev)
        self.kv_scale = host["kv_scale"].to(dev)
        self.q_out = torch.empty(T, H, 576, dtype=torch.float8_e4m3fn, device=dev)
        self.flags = M.ROPE | M.Q_FP8 | M.KV_FP8
        self.side = torch.cuda.Stream(device=dev)          # default priority

    def _kv(self, qkv):
        kv_c = torch.nn.functional.rms_norm(qkv[:, 1536:2048], (512,), self.g_kv, 1e-6)
        return kv_c, qkv[:, 2048:]

    def _q_b(self, qkv):
        q_a = torch.nn.functional.rms_norm(qkv[:, :1536], (1536,), self.g_q, 1e-6)
        return (q_a @ self.w_qb).view(self.T, self.H, 192)

    def _q(self, qkv):
        q = self._q_b(qkv)
        ql = torch.bmm(q[..., :128].transpose(0, 1).contiguous(), self.w_uk)   # [H, T, 512]
        return ql.transpose(0, 1), q[..., 128:]

    def fused_inputs(self):
        """q_nope, q_pe (views of the q_b output), kv_c and k_pe."""
        qkv = self.hidden @ self.w_a
        kv_c, k_pe = self._kv(qkv)
        q = self._q_b(qkv)
        return q[..., :128], q[..., 128:], kv_c, k_pe

    def producers(self):
        qkv = self.hidden @ self.w_a
        kv_c, k_pe = self._kv(qkv)
        ql_nope, q_pe = self._q(qkv)
        return ql_nope, q_pe, kv_c, k_pe

    def _epilogue(self, ql_nope, q_pe, kv_c, k_pe, extra: int = 0):
        M.mla_decode_q_concat_kv_insert(self.q_out, ql_nope, q_pe, kv_c, k_pe, self.cache,
                                        self.slots, self.positions, self.table, self.q_scale,
                                        self.kv_scale, self.flags | extra)

    def step(self, epilogue: bool = True, copies: bool = False, fork: bool = False,
             fused: bool = False):
        if fused:
            q_nope, q_pe, kv_c, k_pe = self.fused_inputs()
            if epilogue:
                M.mla_decode_uk_q_concat_kv_insert(self.q_out, q_nope, self.w_uk_t, q_pe, kv_c, k_pe,
                                                   self.cache, self.slots, self.positions, self.table,
                                                   self.q_scale, self.kv_scale, self.flags)
            return
        if fork:
            main = torch.cuda.current_stream()
            qkv = self.hidden @ self.w_a
            kv_c, k_pe = self._kv(qkv)
            self.side.wait_stream(main)           # the side branch needs kv_c and k_pe only
            ql_nope, q_pe = self._q(qkv)
            with torch.cuda.stream(self.side):
                self._epilogue(ql_nope, q_pe, kv_c, k_pe, M.CACHE_ROWS_ONLY)
            kv_c.record_stream(self.side)
            k_pe.record_stream(self.side)
            self._epilogue(ql_nope, q_pe, kv_c, k_pe, M.Q_ROWS_ONLY)
            main.wait_stream(self.side)
            return
        ql_nope, q_pe, kv_c, k_pe = self.producers()
        if not epilogue:
            return
        if copies:
            ql_nope, q_pe = ql_nope.contiguous(), q_pe.contiguous()
            kv_c, k_pe = kv_c.contiguous(), k_pe.contiguous()
        self._epilogue(ql_nope, q_pe, kv_c, k_pe)


class DecodeStep(DecodeSlice):
    """The slice above followed by the decode attention that consumes its
    output: B sequences each gain one token (T = B) at position L - 1, the
    epilogue writes that token's E4M3 latent row into the paged cache at its
    slot and its E4M3 query rows, and the attention reads the B queries over
    all L cached rows of each sequence (the other L - 1 rows are synthetic
    E4M3 context)."""

    def __init__(self, B: int, H: int, L: int, dev: str, seed: int = 3):
        super().__init__(B, H, dev, seed)
        w = I.attn_custom(B, H, L, q_fp8=True, kv_fp8=True, name="decode_step")
        host = I.make_attn_inputs(w, seed)
        self.w = w
        self.cache = host["cache"].to(dev)
        self.block_table = host["block_table"].to(dev)
        self.seq_lens = host["seq_lens"].to(dev)
        last = L - 1
        bt = host["block_table"]
        self.slots = (bt[:, last // w.block_size].to(torch.int64) * w.block_size
                      + last % w.block_size).to(dev)
        self.positions = torch.full((B,), last, dtype=torch.int64, device=dev)
        self.out = torch.empty(B, H, 512, dtype=torch.bfloat16, device=dev)
        self.attn = M.PreparedAttention(self.out, self.q_out, self.cache, self.block_table,
                                        self.seq_lens, w.sm_scale, self.q_scale, self.kv_scale,
                                        max_seq_len=L)

    def step(self, epilogue: bool = True, copies: bool = False, attention: bool = True,
             fork: bool = False, fused: bool = False):
        super().step(epilogue, copies, fork, fused)
        if (epilogue or fork) and attention:
            self.attn()


def time_graph_fn(fn, calls: int = 20, replays: int = 20) -> float:
    """Device µs per call of fn when `calls` calls are captured in one graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (calls * replays)


def _alternating_medians(fns: dict, calls: int, rounds: int = 3) -> dict:
    """Graph-replayed µs per call of each fn, the variants measured in turn
    `rounds` times (so that clock and thermal drift hit all alike); the
    median of the rounds per variant."""
    runs = {k: [] for k in fns}
    settle(list(fns.values()), ms=30.0)
    for _ in range(rounds):
        for k, fn in fns.items():
            runs[k].append(time_graph_fn(fn, calls=calls))
    return {k: float(np.median(v)) for k, v in runs.items()}


def decode_slice_timings(dev: str) -> dict:
    """Graph-replayed µs per decode-step slice: producers alone, producers +
    epilogue on strided views, producers + copies + epilogue, and the
    epilogue forked (cache rows on a second stream beside the q_b and W_UK
    products, query rows after them); and the whole step with the decode
    attention over 4096 cached tokens per sequence, unforked and forked."""
    out = {}
    for T in (1, 64, 128):
        ds = DecodeSlice(T, 16, dev)

        def forced(f):
            def run():
                saved = ds.flags
                ds.flags |= f
                ds.step()
                ds.flags = saved
            return run
        r = _alternating_medians({"base": lambda: ds.step(epilogue=False),
                                  "strided": lambda: ds.step(),
                                  "small": forced(M.FORCE_SMALL_T),
                                  "mid": forced(M.FORCE_MID_T),
                                  "copies": lambda: ds.step(copies=True),
                                  "forked": lambda: ds.step(fork=True),
                                  "no_uk": lambda: ds.step(epilogue=False, fused=True),
                                  "fused": lambda: ds.step(fused=True)}, calls=20)
        out[f"t{T}_h16"] = {"producers_us": round(r["base"], 3),
                            "with_epilogue_us": round(r["strided"], 3),
                            "with_copies_and_epilogue_us": round(r["copies"], 3),
                            "with_forked_epilogue_us": round(r["forked"], 3),
                            "producers_before_w_uk_us": round(r["no_uk"], 3),
                            "with_fused_w_uk_epilogue_us": round(r["fused"], 3),
                            "w_uk_and_epilogue_separate_us": round(r["strided"] - r["no_uk"], 3),
                            "w_uk_and_epilogue_fused_us": round(r["fused"] - r["no_uk"], 3),
                            "epilogue_increment_us": round(r["strided"] - r["base"], 3),
                            "epilogue_increment_small_t_us": round(r["small"] - r["base"], 3),
                            "epilogue_increment_mid_t_us": round(r["mid"] - r["base"], 3),
                            "forked_epilogue_increment_us": round(r["forked"] - r["base"], 3),
                            "copies_avoided_us": round(r["copies"] - r["strided"], 3)}
        log(f"decode slice T={T}: {out[f't{T}_h16']}")
    for B in (1, 64):
        st = DecodeStep(B, 16, 4096, dev)
        r = _alternating_medians({"base": lambda: st.step(epilogue=False),
                                  "epi": lambda: st.step(attention=False),
                                  "full": lambda: st.step(),
                                  "forked": lambda: st.step(fork=True),
                                  "fused": lambda: st.step(fused=True)}, calls=10)
        out[f"b{B}_h16_l4096_with_attention"] = {
            "producers_us": round(r["base"], 3), "with_epilogue_us": round(r["epi"], 3),
            "with_epilogue_and_attention_us": round(r["full"], 3),
            "forked_with_attention_us": round(r["forked"], 3),
            "fused_w_uk_epilogue_with_attention_us": round(r["fused"], 3),
            "attention_increment_us": round(r["full"] - r["epi"], 3)}
        log(f"decode step B={B} L=4096: {out[f'b{B}_h16_l4096_with_attention']}")
        del st
    return out


class UkSet:
    """Device copies of one fused-product input set (make_uk_inputs) and
    its prepared call: q_nope and q_pe as views of q_b, as in a step."""

    def __init__(self, w: I.Workload, host: dict, dev: str):
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in host.items()
             if k not in ("q_nope", "q_pe")}
        self.d = d
        qdt = torch.float8_e4m3fn if w.q_fp8 else w.torch_dtype
        self.q_out = torch.empty(w.tokens, w.heads, 576, dtype=qdt, device=dev)
        q_b = d["q_b"]
        self.call = M.PreparedUkInsert(self.q_out, q_b[..., :128], d["w_uk_t"], q_b[..., 128:], d["kv_c"],
                                       d["k_pe"], d["cache"], d["slot_mapping"], d["positions"],
                                       d["rope_cos_sin"], d["q_scale"], d["kv_scale"], flags_of(w))


def _rotating(fns: list):
    """One call of the next of fns in turn (captured several times in a
    graph, the calls walk through the sets)."""
    i = [0]

    def run():
        fns[i[0] % len(fns)]()
        i[0] += 1
    return run


def uk_cpu_oracle(w: I.Workload, host: dict, seconds: float) -> dict:
    """The oracle as it stands for the fused call on the first tokens of the
    workload (as many 64-token chunks as fit in about `seconds`), scaled to
    the whole call: the exact product (fp64), its encoding into q codes, and
    the epilogue oracle for the tails and the cache rows, on all host
    threads."""
    import numpy as np
    import oracle

    def bits(t):
        t = t.contiguous()
        return (t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16)
                else t.view(torch.uint8).numpy())
    T, H = w.tokens, w.heads
    q_nope, q_pe = bits(host["q_nope"]), bits(host["q_pe"])
    kv_c, k_pe, w_uk = bits(host["kv_c"]), bits(host["k_pe"]), bits(host["w_uk_t"])
    cache = bits(host["cache"]).copy()
    slots = host["slot_mapping"].numpy()
    pos = host["positions"].numpy() if host["positions"] is not None else None
    table = host["rope_cos_sin"].numpy() if host["rope_cos_sin"] is not None else None
    done, t0 = 0, time.perf_counter()
    while done < T and time.perf_counter() - t0 < seconds:
        t1 = min(T, done + 64)
        x = oracle.uk_product(q_nope[done:t1], w_uk).astype(np.float32)
        if w.q_fp8:
            q = np.zeros((t1 - done, H, 576), dtype=np.uint8)
            lat = oracle.quant_e4m3_array(x, w.q_scale).reshape(x.shape)
        else:
            q = np.zeros((t1 - done, H, 576), dtype=np.uint16)
            lat = oracle.f32_to_bf16_array(x).reshape(x.shape)
        oracle.insert(q, np.zeros((t1 - done, H, 512), dtype=np.uint16), q_pe[done:t1], kv_c[done:t1],
                      k_pe[done:t1], cache, slots[done:t1], None if pos is None else pos[done:t1], table,
                      w.q_scale, w.kv_scale, w.rope, w.q_fp8, w.kv_fp8)
        q[..., :512] = lat
        done = t1
    el = time.perf_counter() - t0
    return {"us_per_call": round(el / done * T * 1e6, 1), "sample": f"{done} of {T} tokens",
            "kind": "oracle", "cores": oracle.num_threads()}


def uk_timings(dev: str, cpu_seconds: float = 0.0) -> dict:
    """The epilogue fused into the W_UK product, alone, on each workload's
    shapes and flags (inputs from make_uk_inputs): graph-replayed µs per
    call on one buffer set (warm) and, for the two large shapes, on 4
    rotating sets (cold), with GB/s against the call's algorithmic bytes
    (q_nope and W_UK instead of ql_nope) and the product's TFLOP/s; with
    ``cpu_seconds`` the oracle timed beside it on the 8192-token shape."""
    out = {}
    for name in LATENCY + MID + [HEADLINE]:
        w = I.WORKLOADS[name]
        host = I.make_uk_inputs(w)
        nsets = 4 if name in MID + [HEADLINE] else 1
        sets = [UkSet(w, host, dev) for _ in range(nsets)]
        p = M.uk_plan(M._binding._dims(host["q_nope"], host["q_pe"], host["kv_c"], host["k_pe"],
                                       host["cache"], host["rope_cos_sin"]), flags_of(w))
        settle([s.call for s in sets], ms=20.0)
        warm = time_graph_fn(sets[0].call, calls=20 if nsets == 1 else 8)
        r = {"us_per_call_graph": round(warm, 3), "bytes": p.bytes,
             "gbs_graph": round(p.bytes / warm / 1e3, 1),
             "tflops_graph": round(p.flops / warm / 1e6, 2),
             "configuration": "throughput" if p.mapping else "latency",
             "streaming": bool(p.streaming), "grid_blocks": p.grid_blocks}
        if nsets > 1:
            cold = time_graph_fn(_rotating([s.call for s in sets]), calls=8)
            r.update(us_per_call_graph_4_sets=round(cold, 3), gbs_graph_4_sets=round(p.bytes / cold / 1e3, 1))
        if cpu_seconds > 0 and name == HEADLINE:
            r["cpu_oracle"] = uk_cpu_oracle(w, host, cpu_seconds)
        out[name] = r
        log(f"fused W_UK epilogue {name}: {r}")
        del sets
        torch.cuda.empty_cache()
    return out


def attn_algorithmic_bytes(w: I.AttnWorkload) -> int:
    """Bytes decode attention must move per call: every cached row of every
    sequence read once (576 elements), the queries read and the bf16
    outputs written once, the block-table entries in use and the lengths."""
    kv = 1 if w.kv_fp8 else 2
    q = 1 if w.q_fp8 else 2
    rows = sum(w.seq_lens)
    pages = sum((L + w.block_size - 1) // w.block_size for L in w.seq_lens)
    return rows * 576 * kv + w.batch * w.heads * (576 * q + 512 * 2) + pages * 4 + w.batch * 4


def attn_sources_digest() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_traffic_entry(name: str):
    """Measured HBM bytes per call (the partial kernel and its range merge) from the
    committed counter summary, if taken on the current attention sources."""
    if not os.path.exists(ATTN_TRAFFIC_FILE):
        return None
    with open(ATTN_TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("sources_digest") != attn_sources_digest():
        return None
    return t.get("workloads", {}).get(name, {}).get("hbm_bytes_per_call")


def attn_range_kernel(w: I.AttnWorkload, pl) -> str:
    """Which range kernel the plan runs: the loader/compute ring (E4M3 cache),
    its loader-free form for 64-key ranges, or the bf16-cache kernel."""
    if not w.kv_fp8:
        return "mla_attn_partial_kernel"
    return "mla_attn_short_kernel" if pl.keys_per_split == 64 else "mla_attn_ring_kernel"


def attn_plan_for(w: I.AttnWorkload):
    d = M.AttnDims()
    d.batch, d.num_heads, d.num_blocks, d.block_size = w.batch, w.heads, w.num_blocks, w.block_size
    d.max_blocks_per_seq, d.max_seq_len = w.max_blocks, max(w.seq_lens)
    return M.attn_plan(d, (M.ATTN_Q_FP8 if w.q_fp8 else 0) | (M.ATTN_KV_FP8 if w.kv_fp8 else 0))


class AttnSet:
    """One device-resident batch (queries, cache, tables, output) of a
    decode-attention workload, bound to the library call."""

    def __init__(self, w: I.AttnWorkload, host: dict, dev: str):
        self.t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in host.items()}
        t = self.t
        self.out = torch.empty(w.batch, w.heads, 512, dtype=torch.bfloat16, device=dev)
        self.prepared = M.PreparedAttention(self.out, t["q"], t["cache"], t["block_table"],
                                            t["seq_lens"], w.sm_scale, t["q_scale"],
                                            t["kv_scale"], max_seq_len=max(w.seq_lens))

    def call(self):
        self.prepared()


def attn_cpu_oracle(w: I.AttnWorkload, host: dict, seconds: float) -> dict:
    """The float64 attention oracle as it stands, on the first sequences of
    the workload (as many as fit in about `seconds`), scaled to the whole
    batch."""
    import numpy as np
    from oracle import attention as A

    def bits(t):
        t = t.contiguous()
        return (t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16
                else t.view(torch.uint8).numpy())
    q, cache = bits(host["q"]), bits(host["cache"])
    bt, lens = host["block_table"].numpy(), host["seq_lens"].numpy()
    done, t0 = 0, time.perf_counter()
    while done < w.batch and time.perf_counter() - t0 < seconds:
        A.mla_decode_attention(q[done:done + 1], cache, bt[done:done + 1], lens[done:done + 1],
                               w.sm_scale, w.q_scale if w.q_fp8 else None,
                               w.kv_scale if w.kv_fp8 else None)
        done += 1
    el = time.perf_counter() - t0
    per_call_us = el / done * w.batch * 1e6
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    return {"us_per_call": round(per_call_us, 1), "sample": f"{done} of {w.batch} sequences",
            "kind": "oracle", "cores": cores}


def attention_timings(dev: str, steps: int, cpu_seconds: float = 0.0) -> dict:
    """Decode attention over the paged latent cache, per workload: device
    time per call (events around back-to-back calls on the launch stream),
    with enough independent cache copies rotated that their total exceeds
    twice the 256 MB MALL (cold), and with one copy (warm); also the cold
    rotation captured in a HIP graph and replayed (no host launch gaps)."""
    out = {}
    for name, w in I.ATTN_WORKLOADS.items():
        host = I.make_attn_inputs(w)
        cache_bytes = host["cache"].numel() * host["cache"].element_size()
        n_cold = max(1, min(8, -(-(600 << 20) // cache_bytes)))
        sets = [AttnSet(w, host, dev) for _ in range(n_cold)]
        torch.cuda.synchronize()
        calls = max(20, steps // 4)
        settle([s.call for s in sets], ms=60.0)
        cold = time_calls(sets, calls, 5)
        warm = time_calls(sets[:1], calls, 5)
        graph_cold_us = time_graph(sets, calls=10 * len(sets), replays=10)
        nb = attn_algorithmic_bytes(w)
        pl = sets[0].prepared.plan
        out[name] = {
            "config": w.describe(), "bytes": nb, "cold_sets": n_cold,
            "us_per_call": round(cold["event_ms_per_call"] * 1e3, 3),
            "gbs": round(nb / cold["event_ms_per_call"] / 1e6, 1),
            "pct_of_hbm_peak": round(100.0 * nb / cold["event_ms_per_call"] / 1e6 / HBM_PEAK_GBS, 2),
            "us_per_call_graph": round(graph_cold_us, 3),
            "us_per_call_warm": round(warm["event_ms_per_call"] * 1e3, 3),
            "gbs_warm": round(nb / warm["event_ms_per_call"] / 1e6, 1),
            "splits": pl.splits, "keys_per_split": pl.keys_per_split,
            "range_kernel": attn_range_kernel(w, pl), "block_threads": pl.block_threads,
            "workgroups": pl.workgroups, "combine": bool(pl.combine),
            "traffic_bytes": attn_traffic_entry(name),
        }
        if cpu_seconds > 0:
            out[name]["cpu_oracle"] = attn_cpu_oracle(w, host, cpu_seconds)
        log(f"attention {name}: {out[name]}")
        del sets
        torch.cuda.empty_cache()
    return out


def sources_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(bytes_per_launch: int):
    """Measured HBM bytes per launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("sources_digest") != sources_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w: I.Workload, host: dict, budget_s: float) -> dict:
    """The CPU oracle, as it stands, on the same workload's host arrays."""
    import numpy as np
    import oracle

    def bits(t):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.view(torch.uint8).numpy()

    T, H = w.tokens, w.heads
    q = np.zeros((T, H, I.ROW), dtype=np.uint8 if w.q_fp8 else np.uint16)
    cache = bits(host["cache"]).copy()
    args = (q, bits(host["ql_nope"]), bits(host["q_pe"]), bits(host["kv_c"]), bits(host["k_pe"]),
            cache, host["slot_mapping"].numpy(),
            host["positions"].numpy() if host["positions"] is not None else None,
            host["rope_cos_sin"].numpy() if host["rope_cos_sin"] is not None else None,
            w.q_scale, w.kv_scale, w.rope, w.q_fp8, w.kv_fp8)
    def timed(seconds):
        oracle.insert(*args)                  # warm-up (page faults, thread start)
        runs = 0
        t0 = time.perf_counter()
        while True:
            oracle.insert(*args)
            runs += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return (time.perf_counter() - t0) / runs, runs

    cores = oracle.num_threads()
    dt, runs = timed(budget_s)
    oracle.set_num_threads(1)
    dt1, runs1 = timed(budget_s / 3)
    oracle.set_num_threads(cores)
    nb = algorithmic_bytes(w)
    return {"value": round(nb / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"full {w.name} workload ({w.describe()}), {runs} calls after 1 warm-up, "
                      f"{dt * 1e3:.1f} ms per call",
            "single_thread": {"value": round(nb / dt1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "sample": f"{runs1} calls, {dt1 * 1e3:.1f} ms per call"}}


def copy_reference(dev: str, moved_bytes: int, calls: int = 50) -> dict:
    """The runtime's own device copy (torch copy_, a blit kernel) moving the
    same number of bytes as one headline call (half read, half written), on
    four rotating buffer pairs like the headline: a practical HBM ceiling for
    a read+write stream on this GPU, measured beside the epilogue."""
    n = (moved_bytes // 2) // 4096 * 4096
    pairs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(1),
              torch.empty(n, dtype=torch.uint8, device=dev)) for _ in range(4)]
    for i in range(8):
        pairs[i % 4][1].copy_(pairs[i % 4][0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        pairs[i % 4][1].copy_(pairs[i % 4][0])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    del pairs
    torch.cuda.empty_cache()
    return {"what": "torch copy_ of the same bytes (runtime blit kernel), 4 rotating pairs",
            "bytes_moved": 2 * n, "us_per_call": round(us, 3), "gbs": round(2 * n / us / 1e3, 1)}


# (name, tokens or sequences, cached tokens (None: the slice without the
# attention), step mode ("one": one epilogue launch after the W_UK product,
# "forked": cache rows on a second stream, "fused": W_UK product and epilogue
# in one launch), extra epilogue flags, epilogue alone on the slice's views)
STEP_TRACE_CASES = [
    ("slice_t64_h16", 64, None, "one", 0, False),
    ("slice_t64_h16_mid_t", 64, None, "one", M.FORCE_MID_T, False),
    ("slice_t64_h16_epilogue_alone", 64, None, "one", 0, True),
    ("slice_t64_h16_forked", 64, None, "forked", 0, False),
    ("slice_t64_h16_fused", 64, None, "fused", 0, False),
    ("step_b64_h16_l4096", 64, 4096, "one", 0, False),
    ("step_b64_h16_l4096_forked", 64, 4096, "forked", 0, False),
    ("step_b64_h16_l4096_fused", 64, 4096, "fused", 0, False),
    ("step_b1_h16_l4096", 1, 4096, "one", 0, False),
    ("step_b1_h16_l4096_forked", 1, 4096, "forked", 0, False),
    ("step_b1_h16_l4096_fused", 1, 4096, "fused", 0, False),
]


def step_trace(dev: str, replays: int) -> None:
    """For a kernel trace of one decode step: each case captures ONE step in
    a HIP graph (or only its epilogue, on views the producers wrote once)
    and replays it `replays` times, draining the GPU and idling 200 µs
    between replays, so that in the trace every replay is a group of kernels
    set apart by idle time (see trace_summary)."""
    for name, T, L, mode, extra, alone in STEP_TRACE_CASES:
        obj = DecodeSlice(T, 16, dev) if L is None else DecodeStep(T, 16, L, dev)
        obj.flags |= extra
        if alone:
            views = obj.producers()
            fn = lambda: obj._epilogue(*views)           # noqa: E731
        else:
            fn = lambda: obj.step(fork=mode == "forked", fused=mode == "fused")   # noqa: E731
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(replays):
            g.replay()
            torch.cuda.synchronize()
            time.sleep(200e-6)
        log(f"step trace {name}: {replays} replays")
        del g, obj, fn
        torch.cuda.empty_cache()


def _short_kernel_name(name: str) -> str:
    if name.startswith("Cijk_") or "gemm" in name.lower():
        return "GEMM (hipBLASLt)"
    for key in ("mla_dq_epilogue_kernel", "mla_dq_uk_epilogue_kernel", "mla_attn_ring_kernel",
                "mla_attn_short_kernel", "mla_attn_partial_kernel",
                "mla_attn_combine_wide_kernel", "mla_attn_combine_kernel"):
        if key in name:
            return key
    if "rms_norm" in name.lower() or "rmsnorm" in name.lower() or "layer_norm" in name.lower():
        return "RMSNorm (torch)"
    if "elementwise" in name or "copy" in name.lower():
        return "elementwise (torch)"
    return name[:40]


def trace_summary(csv_path: str, idle_us: float = 100.0) -> str:
    """Median timeline of the replayed steps in a rocprofv3 kernel trace.

    Kernels are split into replays at idle gaps longer than ``idle_us``;
    replays with the same kernel sequence (name and grid) form one case.
    For each case and kernel: median start and end relative to the replay's
    first kernel start, median duration, and the median gap from the latest
    end of the kernels before it (negative: it overlaps one of them)."""
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         _short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]),
                         int(r["Workgroup_Size_X"])))
    rows.sort()
    groups, cur = [], []
    for r in rows:
        if cur and r[0] - max(x[1] for x in cur) > idle_us * 1e3:
            groups.append(cur)
            cur = []
        cur.append(r)
    if cur:
        groups.append(cur)
    cases = {}
    for g in groups:
        sig = tuple((x[2], x[3] // x[4]) for x in g)
        cases.setdefault(sig, []).append(g)
    # cases in the order they first ran; named after --step-trace's cases
    # when the trace holds exactly those
    kept = sorted(((sig, gs) for sig, gs in cases.items()
                   if len(gs) >= 5 and any(k[0] in ("mla_dq_epilogue_kernel", "mla_dq_uk_epilogue_kernel")
                                           for k in sig)),
                  key=lambda kv: float(np.median([g[0][0] for g in kv[1]])))
    names = [c[0] for c in STEP_TRACE_CASES] if len(kept) == len(STEP_TRACE_CASES) else [""] * len(kept)
    lines = []
    for (sig, gs), name in zip(kept, names):
        title = f"{name}: " if name else ""
        lines.append(f"\n### {title}{len(gs)} replays of {len(sig)} kernels\n")
        lines.append("Median µs from the first kernel's start:\n")
        lines.append("| # | Kernel | Workgroups | Start | End | Duration | Gap from previous end |")
        lines.append("|---|---|---|---|---|---|---|")
        total = []
        for k, (nm, wgs) in enumerate(sig):
            st = [(g[k][0] - g[0][0]) / 1e3 for g in gs]
            en = [(g[k][1] - g[0][0]) / 1e3 for g in gs]
            du = [(g[k][1] - g[k][0]) / 1e3 for g in gs]
            gap = [(g[k][0] - max(x[1] for x in g[:k])) / 1e3 for g in gs] if k else [0.0]
            lines.append(f"| {k} | {nm} | {wgs} | {np.median(st):.2f} | {np.median(en):.2f} | "
                         f"{np.median(du):.2f} | {np.median(gap):.2f} |" if k else
                         f"| {k} | {nm} | {wgs} | {np.median(st):.2f} | {np.median(en):.2f} | "
                         f"{np.median(du):.2f} | — |")
        total = [(max(x[1] for x in g) - g[0][0]) / 1e3 for g in gs]
        busy = [sum(x[1] - x[0] for x in g) / 1e3 for g in gs]
        lines.append(f"\nFirst start to last end: median {np.median(total):.2f} µs; sum of kernel "
                     f"durations {np.median(busy):.2f} µs.")
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=I.WORKLOAD_ORDER)
    ap.add_argument("--buffer-sets", type=int, default=4,
                    help="independent input/output sets rotated between calls (defeats the MALL)")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-decode-slice", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--only-attention", action="store_true",
                    help="time only the decode-attention workloads (prints their JSON)")
    ap.add_argument("--no-uk", action="store_true")
    ap.add_argument("--only-uk", action="store_true",
                    help="time only the epilogue fused into the W_UK product (prints its JSON)")
    ap.add_argument("--only-decode-slice", action="store_true",
                    help="time only the decode-step slices in HIP graphs (prints their JSON)")
    ap.add_argument("--step-trace", type=int, default=0, metavar="REPLAYS",
                    help="replay one captured decode step per case REPLAYS times, apart "
                         "(for a rocprofv3 kernel trace; see --trace-summary)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print the per-replay kernel timeline of a rocprofv3 kernel trace "
                         "(no GPU needed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch copies of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the epilogue exchanges nothing between GPUs, "
              "so it runs and reports a single MI355X (use --gpus 1).", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.step_trace:
        step_trace(dev, args.step_trace)
        return 0
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB x {args.steps}")
        return 0

    M.load()
    if args.only_attention:
        print(json.dumps({"decode_attention": attention_timings(dev, args.steps)}), flush=True)
        return 0
    if args.only_decode_slice:
        print(json.dumps({"decode_step_slice_graph": decode_slice_timings(dev)}), flush=True)
        return 0
    if args.only_uk:
        print(json.dumps({"fused_w_uk_epilogue": uk_timings(dev, 0.0 if args.no_cpu_baseline else 3.0)}),
              flush=True)
        return 0
    w = I.WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.describe()}")
    host = I.make_inputs(w)
    sets = []
    for i in range(max(1, args.buffer_sets)):
        sets.append(DeviceSet(w, host, dev))
    torch.cuda.synchronize()
    log(f"{len(sets)} buffer sets resident; timing {args.steps} steps after {args.warmup} warm-up")
    settle([s.call for s in sets])
    r = time_calls(sets, args.steps, args.warmup)
    nbytes = algorithmic_bytes(w)
    ms = r["wall_ms_per_call"]
    value = nbytes / (ms * 1e-3) / 1e9
    achieved = nbytes / (r["event_ms_per_call"] * 1e-3) / 1e9
    log(f"{r['event_ms_per_call'] * 1e3:.2f} us/launch (events), {achieved:.0f} GB/s")
    pl = M.plan(M.Dims(num_tokens=w.tokens, num_heads=w.heads, num_blocks=w.num_blocks,
                       block_size=w.block_size, max_position=w.max_position), flags_of(w))
    del sets
    torch.cuda.empty_cache()

    latency = {}
    if not args.no_latency:
        # launch floor: the same graph replay of a kernel that writes 4 bytes
        tiny = torch.zeros(1, dtype=torch.float32, device=dev)
        latency["graph_floor_one_element_fill"] = {"us_per_call_graph": round(time_graph_fn(lambda: tiny.fill_(1.0), calls=100), 3)}
        log(f"graph floor (one-element fill): {latency['graph_floor_one_element_fill']}")
        for name in LATENCY:
            lw = I.WORKLOADS[name]
            lh = I.make_inputs(lw)
            one = [DeviceSet(lw, lh, dev)]
            eight = [DeviceSet(lw, lh, dev) for _ in range(8)]
            settle([one[0].call], ms=20.0)
            latency[name] = {
                "us_per_call_graph": round(time_graph(one), 3),
                "us_per_call_graph_8_sets": round(time_graph(eight), 3),
                "us_per_call_queued": round(time_queued(one[0]), 3),
                "host_us_per_call_binding": round(time_host(one[0].call), 3),
                "host_us_per_call_prepared": round(time_host(one[0].prepared), 3),
                "bytes": algorithmic_bytes(lw),
            }
            log(f"{name}: {latency[name]}")
            del one, eight
        for name in MID:
            mw = I.WORKLOADS[name]
            mh = I.make_inputs(mw)
            sets4 = [DeviceSet(mw, mh, dev) for _ in range(4)]
            settle([s.call for s in sets4])
            warm_us = time_graph(sets4[:1], calls=50, replays=10)
            cold_us = time_graph(sets4, calls=50, replays=10)
            nb = algorithmic_bytes(mw)
            latency[name] = {"us_per_call_graph": round(warm_us, 3),
                             "us_per_call_graph_4_sets": round(cold_us, 3),
                             "gbs_graph": round(nb / warm_us / 1e3, 1),
                             "gbs_graph_4_sets": round(nb / cold_us / 1e3, 1), "bytes": nb}
            log(f"{name}: {latency[name]}")
            del sets4

    variants = {}
    if not args.no_variants:
        import dataclasses
        for vname, kw in VARIANTS.items():
            vw = dataclasses.replace(w, name=f"{w.name}_{vname}", **kw)
            vh = I.make_inputs(vw)
            vsets = [DeviceSet(vw, vh, dev) for _ in range(max(1, args.buffer_sets))]
            settle([s.call for s in vsets])
            vr = time_calls(vsets, max(20, args.steps // 4), 5)
            vb = algorithmic_bytes(vw)
            variants[vname] = {"us_per_call": round(vr["event_ms_per_call"] * 1e3, 3),
                               "gbs": round(vb / vr["event_ms_per_call"] / 1e6, 1),
                               "bytes": vb}
            log(f"variant {vname}: {variants[vname]}")
            del vsets
            torch.cuda.empty_cache()

    ref_copy = copy_reference(dev, nbytes)
    log(f"reference copy: {ref_copy}")
    decode_slice = {} if args.no_decode_slice else decode_slice_timings(dev)
    fused_uk = {} if args.no_uk else uk_timings(dev, 0.0 if args.no_cpu_baseline else 3.0)
    attention = {} if args.no_attention else attention_timings(
        dev, args.steps, 0.0 if args.no_cpu_baseline else 3.0)

    traffic = traffic_entry(nbytes)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "heads": w.heads,
                   "cache": f"[{w.num_blocks},{w.block_size},576] {'e4m3' if w.kv_fp8 else 'bf16'}",
                   "q_out": "e4m3" if w.q_fp8 else "bf16", "rope": w.rope,
                   "buffer_sets": args.buffer_sets,
                   "mapping": {0: "small_t", 1: "large_t", 2: "mid_t"}[pl.mapping],
                   "streaming": bool(pl.streaming),
                   "grid_blocks": pl.grid_blocks, "block_threads": pl.block_threads,
                   "rows_per_wave": pl.rows_per_wave, "tail_steps": pl.tail_steps},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "reference_copy": ref_copy,
        "latency_us": latency,
        "variants_at_headline_shape": variants,
        "decode_step_slice_graph": decode_slice,
        "fused_w_uk_epilogue": fused_uk,
        "decode_attention": attention,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "kernel_us": round(r["event_ms_per_call"] * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
