"""CPU oracle for the fused MLA decode epilogue -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code, header, table or constant.

The arithmetic lives in ``mla_oracle.c`` (plain scalar C, fp32 rounding per
operation, no fused multiply-add); this module only compiles it with gcc and
marshals numpy arrays.  What it computes is stated in the C file's header and
follows the prhub summary of vLLM PR #54896 (Kimi-K3 MLA decode kernel),
sections "implementation breakdown" and "key source snippets".

Parity status: every exported function is pinned in ``tests/test_oracle_pins.py``
(format definitions, brute force, closed forms, the page's own identity).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off keeps every product and sum separately rounded.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build() -> str:
    """Compile the oracle into ``oracle/liboracle.so`` (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_quant_e4m3.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.oracle_quant_e4m3.restype = ctypes.c_uint8
    lib.oracle_rope_neox_f32.argtypes = [u16p, f32p, f32p]
    lib.oracle_rope_neox_f32.restype = None
    lib.oracle_rope_neox_f64.argtypes = [u16p, f32p, f64p]
    lib.oracle_rope_neox_f64.restype = None
    lib.oracle_rope_f32.argtypes = [f32p, f32p, f32p, ctypes.c_int, f32p]
    lib.oracle_rope_f32.restype = None
    lib.oracle_rope_f64.argtypes = [f32p, f32p, f32p, ctypes.c_int, f64p]
    lib.oracle_rope_f64.restype = None
    lib.oracle_uk_product.argtypes = [f64p, f64p, u16p, u16p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int]
    lib.oracle_uk_product.restype = None
    lib.oracle_fp16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_fp16_rne.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_fp16_rne.restype = ctypes.c_uint16
    lib.oracle_f32_to_fp16_n.argtypes = [f32p, u16p, ctypes.c_int64]
    lib.oracle_f32_to_fp16_n.restype = None
    lib.oracle_fp16_to_f32_n.argtypes = [u16p, f32p, ctypes.c_int64]
    lib.oracle_fp16_to_f32_n.restype = None
    lib.oracle_mla_decode_ex.argtypes = [
        u8p, u16p, u16p, u16p, u16p, u8p, i64p, i64p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_mla_decode_ex.restype = ctypes.c_int
    lib.oracle_mla_decode_q_concat_kv_insert.argtypes = [
        u8p, u16p, u16p, u16p, u16p, u8p, i64p, i64p, f32p,
        ctypes.c_float, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_mla_decode_q_concat_kv_insert.restype = ctypes.c_int
    for name, outp in (("oracle_f32_to_e4m3_n", u8p), ("oracle_f32_to_bf16_n", u16p)):
        fn = getattr(lib, name)
        fn.argtypes = [f32p, outp, ctypes.c_int64]
        fn.restype = None
    lib.oracle_quant_e4m3_n.argtypes = [f32p, ctypes.c_float, u8p, ctypes.c_int64]
    lib.oracle_quant_e4m3_n.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    return lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---- element encoders (scalar wrappers, for pins) --------------------------

def bf16_to_f32(bits: int) -> float:
    return _load().oracle_bf16_to_f32(int(bits) & 0xFFFF)


def f32_to_bf16(x: float) -> int:
    return int(_load().oracle_f32_to_bf16_rne(float(x)))


def f32_to_e4m3(x: float) -> int:
    return int(_load().oracle_f32_to_e4m3(float(x)))


def quant_e4m3(x: float, inv: float) -> int:
    return int(_load().oracle_quant_e4m3(float(x), float(inv)))


def f32_to_bf16_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    _load().oracle_f32_to_bf16_n(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f32_to_e4m3_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint8)
    _load().oracle_f32_to_e4m3_n(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint8), x.size)
    return out


def quant_e4m3_array(x: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of x under a per-tensor scale (inv = fl32(1/scale))."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    inv = float(np.float32(1.0) / np.float32(scale))
    out = np.empty(x.size, dtype=np.uint8)
    _load().oracle_quant_e4m3_n(_ptr(x, ctypes.c_float), inv, _ptr(out, ctypes.c_uint8), x.size)
    return out


def f32_to_fp16_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    _load().oracle_f32_to_fp16_n(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def fp16_to_f32_array(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    out = np.empty(b.size, dtype=np.float32)
    _load().oracle_fp16_to_f32_n(_ptr(b, ctypes.c_uint16), _ptr(out, ctypes.c_float), b.size)
    return out


# ---- rotation -----------------------------------------------------------------

def rope_f32(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray, gptj: bool) -> np.ndarray:
    """fp32 rotation of one 64-wide tail of fp32 values by 32 cos/sin values;
    NeoX pairing (i, i+32) or, with gptj, interleaved pairing (2i, 2i+1)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(cos_row, dtype=np.float32)
    s = np.ascontiguousarray(sin_row, dtype=np.float32)
    assert x.size == 64 and c.size == 32 and s.size == 32
    y = np.empty(64, dtype=np.float32)
    _load().oracle_rope_f32(_ptr(x, ctypes.c_float), _ptr(c, ctypes.c_float),
                            _ptr(s, ctypes.c_float), int(gptj), _ptr(y, ctypes.c_float))
    return y


def rope_f64(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray, gptj: bool) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(cos_row, dtype=np.float32)
    s = np.ascontiguousarray(sin_row, dtype=np.float32)
    y = np.empty(64, dtype=np.float64)
    _load().oracle_rope_f64(_ptr(x, ctypes.c_float), _ptr(c, ctypes.c_float),
                            _ptr(s, ctypes.c_float), int(gptj), _ptr(y, ctypes.c_double))
    return y


def rope_neox_f32(x_bits: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
    """fp32 NeoX rotation of one 64-wide bf16 tail (bits) by one table row."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    cs = np.ascontiguousarray(cs_row, dtype=np.float32)
    assert x.size == 64 and cs.size == 64
    y = np.empty(64, dtype=np.float32)
    _load().oracle_rope_neox_f32(_ptr(x, ctypes.c_uint16), _ptr(cs, ctypes.c_float),
                                 _ptr(y, ctypes.c_float))
    return y


def rope_neox_f64(x_bits: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    cs = np.ascontiguousarray(cs_row, dtype=np.float32)
    y = np.empty(64, dtype=np.float64)
    _load().oracle_rope_neox_f64(_ptr(x, ctypes.c_uint16), _ptr(cs, ctypes.c_float),
                                 _ptr(y, ctypes.c_double))
    return y


# ---- the absorbed key projection (for the epilogue fused into it) ----------

def uk_product(q_nope: np.ndarray, w_uk_t: np.ndarray, fp16: bool = False,
               with_mag: bool = False):
    """ql[t,h,n] = sum_k q_nope[t,h,k] * w_uk_t[h,n,k], evaluated in double.

    q_nope [T, H, 128] and w_uk_t [H, 512, 128] are bf16 (or fp16) bit
    patterns (uint16).  Returns float64 [T, H, 512]; with ``with_mag`` also
    sum_k |q_nope[t,h,k] * w_uk_t[h,n,k]|, the scale of any fp32 evaluation's
    rounding error."""
    q = np.ascontiguousarray(q_nope, dtype=np.uint16)
    w = np.ascontiguousarray(w_uk_t, dtype=np.uint16)
    T, H = q.shape[0], q.shape[1]
    assert q.shape == (T, H, 128) and w.shape == (H, 512, 128)
    out = np.empty((T, H, 512), dtype=np.float64)
    mag = np.empty((T, H, 512), dtype=np.float64) if with_mag else None
    _load().oracle_uk_product(_ptr(out, ctypes.c_double),
                              _ptr(mag, ctypes.c_double) if with_mag else None,
                              _ptr(q, ctypes.c_uint16), _ptr(w, ctypes.c_uint16), T, H, int(fp16))
    return (out, mag) if with_mag else out


# ---- the whole epilogue ---------------------------------------------------

def insert(q_out: np.ndarray, ql_nope: np.ndarray, q_pe: np.ndarray,
           kv_c: np.ndarray, k_pe: np.ndarray, cache: np.ndarray,
           slots: np.ndarray, positions: np.ndarray | None,
           cos_sin: np.ndarray | None, q_scale: float, kv_scale: float,
           rope: bool, q_fp8: bool, kv_fp8: bool, fp16: bool = False,
           gptj: bool = False) -> None:
    """Run the oracle in place.

    Arrays are numpy, contiguous: bf16 or fp16 tensors as uint16 bit
    patterns, E4M3 tensors as uint8 codes.  ``q_out`` is [T, H, 576] (uint16
    or uint8), ``cache`` is [num_blocks, block_size, 576] (uint16 or uint8)
    and is updated in place.  ``cos_sin`` is the [max_position, 64] table as
    float32, or as uint16 bf16 bit patterns.
    """
    T, H = ql_nope.shape[0], ql_nope.shape[1]
    assert ql_nope.shape == (T, H, 512) and q_pe.shape == (T, H, 64)
    assert kv_c.shape == (T, 512) and k_pe.shape == (T, 64)
    assert slots.shape == (T,)
    assert q_out.shape == (T, H, 576)
    assert q_out.dtype == (np.uint8 if q_fp8 else np.uint16)
    assert cache.dtype == (np.uint8 if kv_fp8 else np.uint16)
    assert cache.shape[-1] == 576
    num_slots = cache.size // 576
    for a in (q_out, ql_nope, q_pe, kv_c, k_pe, cache, slots):
        assert a.flags["C_CONTIGUOUS"]
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    table_bf16 = False
    if rope:
        positions = np.ascontiguousarray(positions, dtype=np.int64)
        cos_sin = np.ascontiguousarray(cos_sin)
        assert cos_sin.dtype in (np.float32, np.uint16)
        table_bf16 = cos_sin.dtype == np.uint16
        assert positions.shape == (T,) and cos_sin.ndim == 2 and cos_sin.shape[1] == 64
        max_pos = cos_sin.shape[0]
        pos_p = _ptr(positions, ctypes.c_int64)
        cs_p = cos_sin.ctypes.data_as(ctypes.c_void_p)
    else:
        max_pos = 0
        pos_p = None
        cs_p = None
    rc = _load().oracle_mla_decode_ex(
        q_out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
        _ptr(ql_nope, ctypes.c_uint16), _ptr(q_pe, ctypes.c_uint16),
        _ptr(kv_c, ctypes.c_uint16), _ptr(k_pe, ctypes.c_uint16),
        cache.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
        _ptr(slots, ctypes.c_int64), pos_p, cs_p,
        float(q_scale), float(kv_scale), T, H, num_slots, max_pos,
        int(rope), int(q_fp8), int(kv_fp8), int(fp16), int(gptj), int(table_bf16))
    if rc != 0:
        raise ValueError(f"oracle rejected the shapes (rc={rc})")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the OpenMP loop over tokens (timing only)."""
    _load().oracle_set_num_threads(int(n))
