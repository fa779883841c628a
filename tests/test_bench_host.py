"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind
every GB/s and roofline figure, the per-replay timeline of a kernel trace,
and the refusal of more than one GPU."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import pytest

import bench
import mla_decode_concat_amd as M
from mla_decode_concat_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Algorithmic bytes per call of the five workloads, as the scope's measurement
# table states them (reads + writes).
WORKLOAD_BYTES = {
    "t1_h16_copy": 19_592 + 19_584,
    "t64_h16_rope_fp8": 1_270_784 + 626_688,
    "t65_h16_rope_fp8": 1_290_640 + 636_480,
    "t256_h128_rope_qfp8": 38_113_280 + 19_169_280,
    "t8192_h16_rope_kvfp8": 162_660_352 + 155_713_536,
}


@pytest.mark.parametrize("name", list(WORKLOAD_BYTES))
def test_workload_bytes_match_the_stated_figures_and_the_library(name):
    w = I.WORKLOADS[name]
    assert bench.algorithmic_bytes(w) == WORKLOAD_BYTES[name]
    d = M.Dims(num_tokens=w.tokens, num_heads=w.heads, num_blocks=w.num_blocks, block_size=w.block_size,
               max_position=w.max_position, ql_nope_stride_t=w.heads * 512, ql_nope_stride_h=512,
               q_pe_stride_t=w.heads * 64, q_pe_stride_h=64, kv_c_stride_t=512, k_pe_stride_t=64)
    assert M.plan(d, bench.flags_of(w)).bytes == WORKLOAD_BYTES[name]


def test_attention_bytes():
    """Every cached row read once, queries read and outputs written once,
    the block-table entries in use and the lengths: 64 sequences of 4096
    tokens with 16 heads."""
    e4m3 = I.ATTN_WORKLOADS["attn_b64_l4096_h16_kvfp8"]
    bf16 = I.ATTN_WORKLOADS["attn_b64_l4096_h16_bf16"]
    rows, pages = 64 * 4096, 64 * 64
    assert bench.attn_algorithmic_bytes(e4m3) == rows * 576 + 64 * 16 * (576 * 2 + 1024) + pages * 4 + 64 * 4
    assert bench.attn_algorithmic_bytes(e4m3) == 153_239_808
    assert bench.attn_algorithmic_bytes(bf16) == 304_234_752


def _write_trace(path, replays: int, steps):
    """A rocprofv3-style kernel trace: `replays` groups of the kernels in
    `steps` ((name, workgroups, duration ns, gap ns before it)), the groups
    1 ms apart."""
    t = 1_000_000
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"])
        for _ in range(replays):
            for name, wgs, dur, gap in steps:
                t += gap
                wr.writerow(["KERNEL_DISPATCH", name, t, t + dur, wgs * 256, 256])
                t += dur
            t += 1_000_000


def test_trace_summary_timeline(tmp_path):
    steps = [("Cijk_Ailk_Bljk_BBS_BH_MT64x64", 33, 10_000, 0),
             ("void mla_dq::mla_dq_epilogue_kernel<64, 1, 1>(mla_dq::KernelArgs)", 306, 2_000, 500),
             ("void mla_attn::mla_attn_ring_kernel<false, false, true>(mla_attn::Args)", 256, 30_000, 0)]
    path = tmp_path / "run_kernel_trace.csv"
    _write_trace(path, 6, steps)
    out = bench.trace_summary(str(path))
    assert "6 replays of 3 kernels" in out
    lines = [ln for ln in out.splitlines() if ln.startswith("| ") and not ln.startswith("| #")]
    assert lines[0].split("|")[2].strip() == "GEMM (hipBLASLt)"
    epi = [c.strip() for c in lines[1].split("|")]
    assert epi[2] == "mla_dq_epilogue_kernel" and epi[3] == "306"
    assert epi[4:8] == ["10.50", "12.50", "2.00", "0.50"]          # start, end, duration, gap
    ring = [c.strip() for c in lines[2].split("|")]
    assert ring[2] == "mla_attn_ring_kernel" and ring[4:8] == ["12.50", "42.50", "30.00", "0.00"]
    assert "First start to last end: median 42.50 µs; sum of kernel durations 42.00 µs." in out


def test_attention_range_kernel_names():
    """The name bench.py reports is the kernel the plan launches: 64-key
    ranges on an E4M3 cache take the loader-free kernel (256 threads)."""
    for name, want in (("attn_b64_l4096_h16_kvfp8", "mla_attn_ring_kernel"),
                       ("attn_b1_l1024_h16_kvfp8", "mla_attn_short_kernel"),
                       ("attn_b64_l4096_h16_bf16", "mla_attn_partial_kernel"),
                       ("attn_b256_l4096_h16_kvfp8", "mla_attn_ring_kernel")):
        w = I.ATTN_WORKLOADS[name]
        pl = bench.attn_plan_for(w)
        assert bench.attn_range_kernel(w, pl) == want
        assert pl.block_threads == (512 if want == "mla_attn_ring_kernel" else 256)


def test_trace_kernel_labels():
    assert bench._short_kernel_name("void mla_attn::mla_attn_short_kernel<true, false, false>(mla_attn::Args)") \
        == "mla_attn_short_kernel"
    assert bench._short_kernel_name("void mla_attn::mla_attn_combine_wide_kernel<true>(mla_attn::Args)") \
        == "mla_attn_combine_wide_kernel"
    assert bench._short_kernel_name("Cijk_Ailk_Bljk_BBS_BH_MT64x64") == "GEMM (hipBLASLt)"


def test_trace_summary_drops_cases_without_an_epilogue_and_rare_cases(tmp_path):
    path = tmp_path / "run_kernel_trace.csv"
    _write_trace(path, 6, [("Cijk_only_gemm", 8, 5_000, 0)])
    assert bench.trace_summary(str(path)).strip() == ""
    _write_trace(path, 4, [("void mla_dq::mla_dq_uk_epilogue_kernel<1, 1>(x)", 130, 3_000, 0)])
    assert bench.trace_summary(str(path)).strip() == ""          # fewer than 5 replays


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
