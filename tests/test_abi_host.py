"""Host-side tests of the C ABI (no GPU): the library loads and exports every
function include/mla_dq.h declares, argument validation returns the documented
codes without launching, the launch plan follows the token threshold, and
the device-side fast division is exact."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import mla_decode_concat_amd as M
from mla_decode_concat_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_dq.h")
ATTN_HEADER = os.path.join(ROOT, "include", "mla_attn.h")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == {"mla_decode_q_concat_kv_insert", "mla_dq_strerror", "mla_dq_plan",
                          "mla_dq_source_digest", "mla_decode_uk_q_concat_kv_insert", "mla_dq_uk_plan"}
    lib = ctypes.CDLL(B.library_path())
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTED_SYMBOLS) == set(names)


def test_library_exports_every_attention_function():
    names = _declared_functions(ATTN_HEADER)
    assert set(names) == {"mla_decode_attention", "mla_decode_attention_workspace_size",
                          "mla_decode_attention_plan", "mla_decode_attention_noalloc"}
    lib = ctypes.CDLL(B.library_path())
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.ATTN_EXPORTED_SYMBOLS) == set(names)


def test_flag_and_code_values_match_header():
    text = open(HEADER).read()

    def val(name):
        m = re.search(rf"#define {name}\s+\(?([-\w<\s]+)\)?", text)
        return eval(m.group(1).replace("u", ""))
    assert val("MLA_DQ_ROPE") == M.ROPE and val("MLA_DQ_Q_FP8") == M.Q_FP8
    assert val("MLA_DQ_KV_FP8") == M.KV_FP8
    assert val("MLA_DQ_FORCE_SMALL_T") == M.FORCE_SMALL_T
    assert val("MLA_DQ_FORCE_LARGE_T") == M.FORCE_LARGE_T
    assert val("MLA_DQ_FP16") == M.FP16 and val("MLA_DQ_ROPE_GPTJ") == M.ROPE_GPTJ
    assert val("MLA_DQ_TABLE_BF16") == M.TABLE_BF16
    assert val("MLA_DQ_FORCE_STREAM") == M.FORCE_STREAM
    assert val("MLA_DQ_FORCE_CACHED") == M.FORCE_CACHED
    assert val("MLA_DQ_FORCE_MID_T") == M.FORCE_MID_T
    assert val("MLA_DQ_Q_ROWS_ONLY") == M.Q_ROWS_ONLY
    assert val("MLA_DQ_CACHE_ROWS_ONLY") == M.CACHE_ROWS_ONLY
    for name, v in (("MLA_DQ_ERR_NULL", B.ERR_NULL), ("MLA_DQ_ERR_ALIGN", B.ERR_ALIGN),
                    ("MLA_DQ_ERR_DIM", B.ERR_DIM), ("MLA_DQ_ERR_FLAGS", B.ERR_FLAGS),
                    ("MLA_DQ_ERR_LAUNCH", B.ERR_LAUNCH), ("MLA_DQ_ERR_ALIAS", B.ERR_ALIAS)):
        assert int(re.search(rf"#define {name}\s+(-?\d+)", text).group(1)) == v


def test_plan_and_dims_structs_match_header_layout():
    """The ctypes mirrors of mla_dq_launch_plan and mla_dq_dims list the
    header's fields in the header's order and types."""
    import ctypes
    text = open(HEADER).read()
    body = re.search(r"typedef struct mla_dq_launch_plan \{(.*?)\} mla_dq_launch_plan;", text, re.S).group(1)
    fields = re.findall(r"(int32_t|int64_t)\s+(\w+);", body)
    want = [(n, ctypes.c_int32 if t == "int32_t" else ctypes.c_int64) for t, n in fields]
    assert [(n, t) for n, t in B.LaunchPlan._fields_] == want
    body = re.search(r"typedef struct mla_dq_dims \{(.*?)\} mla_dq_dims;", text, re.S).group(1)
    assert [n for n, _ in B.Dims._fields_] == re.findall(r"int64_t\s+(\w+);", body)


def test_strerror_every_code():
    seen = set()
    for c in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = M.strerror(c)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in M.strerror(-99)


# ---- validation (fake, never-dereferenced addresses; nothing launches) -----

BASE = 1 << 36          # fake device addresses, 16-byte aligned, far apart
GAP = 1 << 32


def _dims(T=4, H=2, NB=1, BS=64, maxpos=16):
    d = B.Dims()
    d.num_tokens, d.num_heads, d.num_blocks, d.block_size, d.max_position = T, H, NB, BS, maxpos
    d.ql_nope_stride_t, d.ql_nope_stride_h = H * 512, 512
    d.q_pe_stride_t, d.q_pe_stride_h = H * 64, 64
    d.kv_c_stride_t, d.k_pe_stride_t = 512, 64
    return d


def _ptrs():
    names = ["q_out", "ql_nope", "q_pe", "kv_c", "k_pe", "cache", "slots", "pos", "cs", "qs", "ks"]
    return {n: BASE + i * GAP for i, n in enumerate(names)}


def _call(p, flags, dims):
    return B.load().mla_decode_q_concat_kv_insert(
        p["q_out"], p["ql_nope"], p["q_pe"], p["kv_c"], p["k_pe"], p["cache"], p["slots"],
        p["pos"], p["cs"], p["qs"], p["ks"], ctypes.c_uint32(flags),
        ctypes.byref(dims) if dims is not None else None, None)


def test_null_dims():
    assert _call(_ptrs(), 0, None) == B.ERR_NULL


@pytest.mark.parametrize("flags", [1 << 6, 1 << 15, 1 << 31, M.FORCE_SMALL_T | M.FORCE_LARGE_T,
                                   M.Q_ROWS_ONLY | M.CACHE_ROWS_ONLY,
                                   M.FORCE_SMALL_T | M.FORCE_MID_T, M.FORCE_MID_T | M.FORCE_LARGE_T,
                                   M.FORCE_SMALL_T | M.FORCE_MID_T | M.FORCE_LARGE_T,
                                   M.FORCE_STREAM | M.FORCE_CACHED, M.ROPE_GPTJ, M.TABLE_BF16,
                                   M.ROPE_GPTJ | M.TABLE_BF16 | M.FP16])
def test_bad_flags(flags):
    assert _call(_ptrs(), flags, _dims()) == B.ERR_FLAGS


@pytest.mark.parametrize("field,value", [("num_tokens", -1), ("num_heads", 0), ("num_blocks", 0),
                                         ("block_size", 0), ("ql_nope_stride_t", -8)])
def test_bad_dims(field, value):
    d = _dims()
    setattr(d, field, value)
    assert _call(_ptrs(), 0, d) == B.ERR_DIM


def test_too_many_chunks_for_32bit_indices():
    d = _dims(T=(1 << 31) // (72 * 3) + 1, H=2)
    assert _call(_ptrs(), 0, d) == B.ERR_DIM


def test_rope_needs_table_rows():
    assert _call(_ptrs(), M.ROPE, _dims(maxpos=0)) == B.ERR_DIM


def test_zero_tokens_is_a_no_op_even_with_null_pointers():
    p = {k: None for k in _ptrs()}
    assert _call(p, M.ROPE | M.Q_FP8 | M.KV_FP8, _dims(T=0)) == B.OK


@pytest.mark.parametrize("name", ["q_out", "ql_nope", "q_pe", "kv_c", "k_pe", "cache", "slots"])
def test_null_required_pointer(name):
    p = _ptrs()
    p[name] = None
    assert _call(p, 0, _dims()) == B.ERR_NULL


@pytest.mark.parametrize("flags,name", [(M.ROPE, "pos"), (M.ROPE, "cs"), (M.Q_FP8, "qs"),
                                        (M.KV_FP8, "ks")])
def test_null_pointer_needed_by_flag(flags, name):
    p = _ptrs()
    p[name] = None
    assert _call(p, flags, _dims()) == B.ERR_NULL


def test_optional_pointers_may_be_null_when_unused():
    p = _ptrs()
    for n in ("pos", "cs", "qs", "ks"):
        p[n] = None
    # passes validation, then q_out overlapping the cache is caught before launch
    p["q_out"] = p["cache"]
    assert _call(p, 0, _dims()) == B.ERR_ALIAS


@pytest.mark.parametrize("name,off", [("q_out", 8), ("ql_nope", 2), ("cache", 8), ("slots", 4)])
def test_misaligned_pointer(name, off):
    p = _ptrs()
    p[name] += off
    assert _call(p, 0, _dims()) == B.ERR_ALIGN


@pytest.mark.parametrize("field", ["ql_nope_stride_t", "ql_nope_stride_h", "q_pe_stride_t",
                                   "q_pe_stride_h", "kv_c_stride_t", "k_pe_stride_t"])
def test_misaligned_stride(field):
    d = _dims()
    setattr(d, field, getattr(d, field) + 4)
    assert _call(_ptrs(), 0, d) == B.ERR_ALIGN


def test_unused_strides_unchecked_for_one_token_one_head():
    d = _dims(T=1, H=1)
    d.ql_nope_stride_t = d.q_pe_stride_t = d.kv_c_stride_t = d.k_pe_stride_t = 3
    d.ql_nope_stride_h = d.q_pe_stride_h = 5
    p = _ptrs()
    p["q_out"] = p["cache"]       # reach the alias check: strides passed
    assert _call(p, 0, d) == B.ERR_ALIAS


def test_q_out_overlapping_input_is_rejected():
    p = _ptrs()
    p["q_out"] = p["ql_nope"] + 1024
    assert _call(p, 0, _dims()) == B.ERR_ALIAS


def test_cache_overlapping_input_is_rejected():
    p = _ptrs()
    p["cache"] = p["kv_c"] + 16
    assert _call(p, 0, _dims()) == B.ERR_ALIAS


@pytest.mark.parametrize("name,flags", [("pos", M.ROPE), ("cs", M.ROPE),
                                        ("cs", M.ROPE | M.TABLE_BF16), ("qs", M.Q_FP8),
                                        ("ks", M.KV_FP8)])
@pytest.mark.parametrize("out", ["q_out", "cache"])
def test_output_overlapping_flagged_input_is_rejected(name, flags, out):
    """Positions, the rope table and the scales count as inputs when the flags
    make the kernel read them: an output over any of them is refused."""
    d = _dims(maxpos=16)
    p = _ptrs()
    # the last byte the kernel would read of that input
    last = {"pos": 4 * 8, "cs": 16 * (128 if flags & M.TABLE_BF16 else 256), "qs": 4, "ks": 4}[name] - 1
    p[out] = (p[name] + last) // 16 * 16 - (16 if out == "q_out" else 0)
    assert _call(p, flags, d) == B.ERR_ALIAS


def test_loaded_library_matches_its_sources():
    """The library on disk carries the digest of the sources beside it."""
    from mla_decode_concat_amd import build as BLD
    lib = ctypes.CDLL(B.library_path())
    assert B.library_digest(lib) == BLD.source_digest()
    B.check_digest(lib)


def test_stale_library_is_refused(tmp_path, monkeypatch):
    """A one-byte change in any source changes the digest, and a library
    whose digest differs from the sources' is refused by load()."""
    import shutil
    from mla_decode_concat_amd import build as BLD
    pkg = tmp_path / "mla_decode_concat_amd"
    shutil.copytree(os.path.join(ROOT, "mla_decode_concat_amd", "csrc"), pkg / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    assert BLD.source_digest(str(pkg), str(tmp_path)) == BLD.source_digest()
    for f in BLD.source_files(str(pkg), str(tmp_path)):
        data = open(f, "rb").read()
        open(f, "wb").write(data + b" ")
        assert BLD.source_digest(str(pkg), str(tmp_path)) != BLD.source_digest(), f
        open(f, "wb").write(data)
    lib = ctypes.CDLL(B.library_path())
    with pytest.raises(B.StaleLibraryError):
        B.check_digest(lib, want="0" * 32)
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(BLD, "source_digest", lambda *a, **k: "f" * 32)
    with pytest.raises(B.StaleLibraryError):
        B.load()


# ---- launch plan -------------------------------------------------------------

def _bytes(T, H, flags):
    rope = bool(flags & M.ROPE)
    table = 128 if flags & M.TABLE_BF16 else 256
    read = T * (H * 1152 + 1152 + 8 + (8 + table if rope else 0))
    write = T * 576 * (H * (1 if flags & M.Q_FP8 else 2) + (1 if flags & M.KV_FP8 else 2))
    return read + write


@pytest.mark.parametrize("T,H", [(1, 16), (64, 16), (65, 1), (8192, 16), (256, 128)])
@pytest.mark.parametrize("fl", [0, M.ROPE | M.Q_FP8, M.ROPE | M.KV_FP8 | M.TABLE_BF16])
def test_plan_of_row_subsets(T, H, fl):
    """A launch restricted to the query rows plans T * H rows, one restricted
    to the cache rows T rows; the two move the bytes of a full launch plus
    one more read of each token's position and table row."""
    full = M.plan(_dims(T=T, H=H), fl)
    q = M.plan(_dims(T=T, H=H), fl | M.Q_ROWS_ONLY)
    c = M.plan(_dims(T=T, H=H), fl | M.CACHE_ROWS_ONLY)
    assert (full.total_rows, q.total_rows, c.total_rows) == (T * (H + 1), T * H, T)
    extra = T * (8 + (128 if fl & M.TABLE_BF16 else 256)) if fl & M.ROPE else 0
    assert q.bytes + c.bytes == full.bytes + extra
    for p in (q, c):
        want = 0 if p.total_rows <= p.small_rows_max else (2 if p.total_rows <= p.mid_rows_max else 1)
        assert p.mapping == want
        tails = {0: 8, 2: 16, 1: 64}[p.mapping]
        assert p.tail_blocks == (p.total_rows + tails - 1) // tails
    d = _dims(T=T, H=H)
    with pytest.raises(M.MlaDqError):
        M.plan(d, fl | M.Q_ROWS_ONLY | M.CACHE_ROWS_ONLY)


def test_plan_threshold_and_coverage():
    pl = M.plan(_dims(T=1, H=16), 0)
    assert 0 < pl.small_rows_max <= pl.mid_rows_max
    for T in (1, 2, 52, 53, 63, 64, 65, 135, 136, 214, 215, 256, 301, 302, 8192):
        for H in (1, 16, 128):
            for flags in (0, M.ROPE | M.KV_FP8, M.ROPE | M.Q_FP8 | M.KV_FP8,
                          M.ROPE | M.ROPE_GPTJ | M.TABLE_BF16 | M.FP16):
                pl = M.plan(_dims(T=T, H=H), flags)
                rows = T * (H + 1)
                assert pl.total_rows == rows
                want = 0 if rows <= pl.small_rows_max else (2 if rows <= pl.mid_rows_max else 1)
                assert pl.mapping == want
                assert pl.block_threads == {0: 64, 2: 128, 1: 256}[pl.mapping]
                assert pl.bytes == _bytes(T, H, flags)
                assert pl.streaming == (1 if pl.bytes >= pl.stream_bytes_min else 0)
                assert pl.block_threads % 64 == 0
                # every latent row and every tail covered, no spare workgroup
                lat = pl.block_threads // 64 * pl.rows_per_wave
                assert pl.latent_blocks * lat >= rows > (pl.latent_blocks - 1) * lat
                tails = pl.block_threads // 8 * pl.tail_steps
                assert pl.tail_blocks * tails >= rows > (pl.tail_blocks - 1) * tails
                assert pl.grid_blocks == pl.tail_blocks + pl.latent_blocks
    assert M.plan(_dims(T=1), M.FORCE_LARGE_T).mapping == 1
    assert M.plan(_dims(T=10 ** 5), M.FORCE_SMALL_T).mapping == 0
    assert M.plan(_dims(T=1), M.FORCE_MID_T).mapping == 2
    assert M.plan(_dims(T=10 ** 5), M.FORCE_MID_T).mapping == 2
    assert M.plan(_dims(T=1), M.FORCE_STREAM).streaming == 1
    assert M.plan(_dims(T=10 ** 5, H=128), M.FORCE_CACHED).streaming == 0
    assert M.plan(_dims(T=0), 0).grid_blocks == 0


def test_plan_defaults_match_measured_choice():
    """The 8192-token workload streams on the throughput mapping; the 1, 64
    and 65-token workloads at 16 heads use the 64-thread latency mapping
    (measured fastest after the W_UK product of a decode step up to about
    2600 rows with at most 32 heads), the 256-token full-head one the
    throughput mapping; with 128 heads the 128-thread mapping takes over
    above 896 rows.  All with the default cache policy below 80 MiB."""
    big = M.plan(_dims(T=8192, H=16, NB=4096), M.ROPE | M.KV_FP8)
    assert (big.mapping, big.streaming) == (1, 1)
    for T, H, mapping in ((1, 16, 0), (64, 16, 0), (65, 16, 0), (150, 16, 0), (151, 16, 2),
                          (77, 32, 0), (78, 32, 2), (6, 128, 0), (7, 128, 2), (39, 128, 2),
                          (40, 128, 1), (301, 16, 2), (302, 16, 1)):
        p = M.plan(_dims(T=T, H=H), M.ROPE | M.Q_FP8 | M.KV_FP8)
        assert (p.mapping, p.streaming) == (mapping, 0), (T, H)
        assert p.small_rows_max == (2560 if H <= 32 else 896) and p.mid_rows_max == 5120


def test_plan_rows_per_wave_by_size_and_policy():
    """The throughput mapping moves two latent rows per wavefront for calls
    of 24 to 96 MiB under the default cache policy (the 256-token full-head
    workload), one otherwise."""
    for T, H, fl, want in ((256, 128, M.ROPE | M.Q_FP8, 2), (8192, 16, M.ROPE | M.KV_FP8, 1),
                           (128, 128, M.ROPE | M.Q_FP8, 2), (64, 128, M.ROPE | M.Q_FP8, 1),
                           (512, 128, M.ROPE | M.Q_FP8, 1), (1024, 16, M.ROPE | M.KV_FP8, 2),
                           (256, 128, M.ROPE | M.Q_FP8 | M.FORCE_STREAM, 1),
                           (256, 128, M.ROPE | M.Q_FP8 | M.FORCE_MID_T, 1)):
        p = M.plan(_dims(T=T, H=H, NB=4096), fl)
        in_band = p.mapping == 1 and not p.streaming and (24 << 20) <= p.bytes <= (96 << 20)
        assert p.rows_per_wave == want == (2 if in_band else 1), (T, H, fl)


def test_plan_rejects_bad_input():
    with pytest.raises(M.MlaDqError):
        M.plan(_dims(T=-1), 0)
    with pytest.raises(M.MlaDqError):
        M.plan(_dims(), M.FORCE_SMALL_T | M.FORCE_LARGE_T)


def test_threshold_env_override_in_fresh_process():
    code = ("import mla_decode_concat_amd as M; from mla_decode_concat_amd import _binding as B;"
            "d=B.Dims(); d.num_tokens=1000; d.num_heads=16; d.num_blocks=1; d.block_size=64;"
            "p=M.plan(d,0); print(p.small_rows_max, p.mapping, p.stream_bytes_min, p.streaming,"
            " p.mid_rows_max); d.num_tokens=1500; print(M.plan(d,0).mapping)")
    env = dict(os.environ, MLA_DQ_SMALL_ROWS_MAX="17000", MLA_DQ_MID_ROWS_MAX="30000",
               MLA_DQ_STREAM_BYTES_MIN="1000", PYTHONPATH=ROOT)
    out = subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True, check=True)
    assert out.stdout.split() == ["17000", "0", "1000", "1", "30000", "2"]


# ---- fast division used by the kernel's index decode --------------------------

FASTDIV_CHECK = r"""
#include "fastdiv.h"
#include <stdio.h>
int main() {
    unsigned long long checked = 0;
    for (uint32_t d = 1; d <= 4096; ++d) {
        FastDiv31 f = make_fastdiv31(d);
        for (uint32_t n = 0; n < 70000; ++n) {
            if (fastdiv31(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
            ++checked;
        }
        const uint32_t top = 0x7FFFFFFFu;
        for (uint32_t k = 0; k < 4096; ++k) {
            uint32_t n = top - k * 524287u;
            if (fastdiv31(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
            uint32_t m = (n / d) * d;   /* multiples and their neighbours */
            if (fastdiv31(m, f) != m / d || (m && fastdiv31(m - 1, f) != (m - 1) / d)) {
                printf("FAIL d=%u m=%u\n", d, m); return 1; }
        }
    }
    const uint32_t big[] = {65535u, 65536u, 1000003u, 0x40000000u, 0x7FFFFFFFu};
    for (uint32_t d : big) {
        FastDiv31 f = make_fastdiv31(d);
        for (uint32_t n = 0x7FFFFFFFu; n > 0x7FFFFFFFu - 3000000u; --n)
            if (fastdiv31(n, f) != n / d) { printf("FAIL d=%u n=%u\n", d, n); return 1; }
    }
    printf("OK %llu\n", checked);
    return 0;
}
"""


def test_fastdiv_exact_on_host():
    csrc = os.path.join(ROOT, "mla_decode_concat_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check.cpp")
        exe = os.path.join(d, "check")
        open(src, "w").write(FASTDIV_CHECK)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", csrc, src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout
