"""ctypes binding of libmla_dq.so (the C ABI in include/mla_dq.h).

Argument marshalling only: torch tensors -> device pointers, shapes and
strides -> mla_dq_dims, torch's current HIP stream -> the stream argument.
Every step of the epilogue runs in the library's gfx950 kernel; there is no
fallback.  If the library is missing it is built once; if that fails, or no
GPU is present, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

# Flag bits and return codes of include/mla_dq.h.
ROPE = 1 << 0
Q_FP8 = 1 << 1
KV_FP8 = 1 << 2
FP16 = 1 << 3
ROPE_GPTJ = 1 << 4
TABLE_BF16 = 1 << 5
FORCE_SMALL_T = 1 << 8
FORCE_LARGE_T = 1 << 9
FORCE_STREAM = 1 << 10
FORCE_CACHED = 1 << 11
FORCE_MID_T = 1 << 12
Q_ROWS_ONLY = 1 << 13
CACHE_ROWS_ONLY = 1 << 14

OK = 0
ERR_NULL = -1
ERR_ALIGN = -2
ERR_DIM = -3
ERR_FLAGS = -4
ERR_LAUNCH = -5
ERR_ALIAS = -6

EXPORTED_SYMBOLS = ("mla_decode_q_concat_kv_insert", "mla_dq_strerror", "mla_dq_plan",
                    "mla_dq_source_digest", "mla_decode_uk_q_concat_kv_insert", "mla_dq_uk_plan")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_tokens", "num_heads", "num_blocks", "block_size", "max_position",
        "ql_nope_stride_t", "ql_nope_stride_h", "q_pe_stride_t", "q_pe_stride_h",
        "kv_c_stride_t", "k_pe_stride_t")]


class LaunchPlan(ctypes.Structure):
    _fields_ = [("mapping", ctypes.c_int32), ("streaming", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("rows_per_wave", ctypes.c_int32),
                ("tail_steps", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("small_rows_max", ctypes.c_int64), ("stream_bytes_min", ctypes.c_int64),
                ("bytes", ctypes.c_int64), ("tail_blocks", ctypes.c_int64),
                ("latent_blocks", ctypes.c_int64), ("grid_blocks", ctypes.c_int64),
                ("total_rows", ctypes.c_int64), ("mid_rows_max", ctypes.c_int64)]


class UkLaunchPlan(ctypes.Structure):
    _fields_ = [("mapping", ctypes.c_int32), ("streaming", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("tail_steps", ctypes.c_int32), ("tokens_per_group", ctypes.c_int32)] + [
        (n, ctypes.c_int64) for n in (
            "column_groups", "units", "product_blocks", "tail_blocks", "cache_blocks", "grid_blocks",
            "bytes", "flops", "stream_bytes_min", "large_rows_min")] + [
        ("head_major", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MlaDqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mla_dq error {code}: {msg}")
        self.code = code


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _build.LIB


class StaleLibraryError(RuntimeError):
    """The library on disk was compiled from other sources than those beside it."""


def library_digest(lib: ctypes.CDLL) -> str:
    lib.mla_dq_source_digest.argtypes = []
    lib.mla_dq_source_digest.restype = ctypes.c_char_p
    return lib.mla_dq_source_digest().decode()


def check_digest(lib: ctypes.CDLL, want: str | None = None) -> None:
    """Raise StaleLibraryError unless the library was built from the sources
    now in the package (or from sources with digest ``want``)."""
    want = _build.source_digest() if want is None else want
    got = library_digest(lib)
    if got != want:
        raise StaleLibraryError(
            f"{_build.LIB} was built from sources with digest {got}, but the sources beside it "
            f"have digest {want}: rebuild it (python -m mla_decode_concat_amd.build)")


def load() -> ctypes.CDLL:
    """Load libmla_dq.so, building it first only if it does not exist.  A
    library built from other sources than the ones beside it is refused
    (StaleLibraryError), never used."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        check_digest(lib)
        vp, i64p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.mla_decode_q_concat_kv_insert.argtypes = [
            vp, vp, vp, vp, vp, vp, i64p, i64p, f32p, f32p, f32p, ctypes.c_uint32,
            ctypes.POINTER(Dims), vp]
        lib.mla_decode_q_concat_kv_insert.restype = ctypes.c_int
        lib.mla_dq_strerror.argtypes = [ctypes.c_int]
        lib.mla_dq_strerror.restype = ctypes.c_char_p
        lib.mla_dq_plan.argtypes = [ctypes.POINTER(Dims), ctypes.c_uint32, ctypes.POINTER(LaunchPlan)]
        lib.mla_dq_plan.restype = ctypes.c_int
        lib.mla_decode_uk_q_concat_kv_insert.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i64p, i64p, f32p, f32p, f32p, ctypes.c_uint32,
            ctypes.POINTER(Dims), vp]
        lib.mla_decode_uk_q_concat_kv_insert.restype = ctypes.c_int
        lib.mla_dq_uk_plan.argtypes = [ctypes.POINTER(Dims), ctypes.c_uint32, ctypes.POINTER(UkLaunchPlan)]
        lib.mla_dq_uk_plan.restype = ctypes.c_int
        _lib = lib
        return lib


def strerror(code: int) -> str:
    return load().mla_dq_strerror(int(code)).decode()


def plan(dims: Dims, flags: int) -> LaunchPlan:
    p = LaunchPlan()
    rc = load().mla_dq_plan(ctypes.byref(dims), ctypes.c_uint32(flags), ctypes.byref(p))
    if rc != OK:
        raise MlaDqError(rc, strerror(rc))
    return p


def uk_plan(dims: Dims, flags: int) -> UkLaunchPlan:
    """The launch of the epilogue fused into the W_UK product (dims as for
    the epilogue; the ql_nope strides describe q_nope)."""
    p = UkLaunchPlan()
    rc = load().mla_dq_uk_plan(ctypes.byref(dims), ctypes.c_uint32(flags), ctypes.byref(p))
    if rc != OK:
        raise MlaDqError(rc, strerror(rc))
    return p


def raw_uk_call(q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                rope_cos_sin, q_scale, kv_scale, flags: int, dims: Dims, stream) -> int:
    """Call the fused product's C entry point with integer addresses; returns its code."""
    return load().mla_decode_uk_q_concat_kv_insert(
        q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin,
        q_scale, kv_scale, ctypes.c_uint32(flags), ctypes.byref(dims), stream)


def raw_call(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin,
             q_scale, kv_scale, flags: int, dims: Dims, stream) -> int:
    """Call the C entry point with integer addresses; returns its code."""
    return load().mla_decode_q_concat_kv_insert(
        q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin,
        q_scale, kv_scale, ctypes.c_uint32(flags), ctypes.byref(dims), stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _dims(ql_nope, q_pe, kv_c, k_pe, cache, rope_cos_sin) -> Dims:
    d = Dims()
    d.num_tokens, d.num_heads = ql_nope.shape[0], ql_nope.shape[1]
    d.num_blocks, d.block_size = cache.shape[0], cache.shape[1]
    d.max_position = rope_cos_sin.shape[0] if rope_cos_sin is not None else 0
    d.ql_nope_stride_t, d.ql_nope_stride_h = ql_nope.stride(0), ql_nope.stride(1)
    d.q_pe_stride_t, d.q_pe_stride_h = q_pe.stride(0), q_pe.stride(1)
    d.kv_c_stride_t, d.k_pe_stride_t = kv_c.stride(0), k_pe.stride(0)
    return d


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _check(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def mla_decode_q_concat_kv_insert(q_out: torch.Tensor, ql_nope: torch.Tensor, q_pe: torch.Tensor,
                                  kv_c: torch.Tensor, k_pe: torch.Tensor, cache: torch.Tensor,
                                  slot_mapping: torch.Tensor, positions: torch.Tensor | None = None,
                                  rope_cos_sin: torch.Tensor | None = None,
                                  q_scale: torch.Tensor | None = None,
                                  kv_scale: torch.Tensor | None = None, flags: int = 0,
                                  stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the fused epilogue on ``stream`` (default: torch's current
    stream).  Writes ``q_out`` [T,H,576] and the cache rows at the slots.

    Flags are the MLA_DQ_* bits; the FP8 bits must agree with the dtypes of
    ``q_out`` and ``cache`` (bf16, or float8_e4m3fn / uint8 codes)."""
    _validate_only(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin,
                   q_scale, kv_scale, flags)
    dev = q_out.device
    dims = _dims(ql_nope, q_pe, kv_c, k_pe, cache, rope_cos_sin)
    args = (_ptr(q_out), _ptr(ql_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe), _ptr(cache),
            _ptr(slot_mapping), _ptr(positions), _ptr(rope_cos_sin), _ptr(q_scale), _ptr(kv_scale))
    _launch(args, flags, dims, dev.index, stream)


def _validate_only(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                   rope_cos_sin, q_scale, kv_scale, flags, nope_name: str = "ql_nope",
                   nope_width: int = 512, extra: tuple = ()) -> None:
    """Dtype, shape, layout and device checks the C ABI cannot make.  For the
    fused product the no-position input is q_nope [T, H, 128] and ``extra``
    holds (name, tensor) pairs of further activation-typed inputs (W_UK)."""
    T = ql_nope.shape[0]
    _check(ql_nope.dim() == 3 and ql_nope.shape[2] == nope_width,
           f"{nope_name} must be [T, H, {nope_width}]")
    H = ql_nope.shape[1]
    _check(tuple(q_pe.shape) == (T, H, 64), "q_pe must be [T, H, 64]")
    _check(tuple(kv_c.shape) == (T, 512) and tuple(k_pe.shape) == (T, 64),
           "kv_c must be [T, 512] and k_pe [T, 64]")
    _check(tuple(q_out.shape) == (T, H, 576) and q_out.is_contiguous(),
           "q_out must be a contiguous [T, H, 576] tensor")
    _check(cache.dim() == 3 and cache.shape[2] == 576 and cache.is_contiguous(),
           "cache must be a contiguous [num_blocks, block_size, 576] tensor")
    act = torch.float16 if flags & FP16 else torch.bfloat16
    for name, t in ((nope_name, ql_nope), ("q_pe", q_pe), ("kv_c", kv_c), ("k_pe", k_pe), *extra):
        _check(t.dtype == act, f"{name} must be {act} (flag FP16 selects fp16)")
        _check(t.stride(-1) == 1, f"{name} must have unit inner stride")
    _check(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (T,)
           and slot_mapping.is_contiguous(), "slot_mapping must be a contiguous int64 [T]")
    q_fp8 = bool(flags & Q_FP8)
    kv_fp8 = bool(flags & KV_FP8)
    _check((q_out.dtype in _FP8) == q_fp8 and (q_fp8 or q_out.dtype == act),
           "q_out dtype must be e4m3 with Q_FP8, the activation type without")
    _check((cache.dtype in _FP8) == kv_fp8 and (kv_fp8 or cache.dtype == act),
           "cache dtype must be e4m3 with KV_FP8, the activation type without")
    if flags & ROPE:
        _check(positions is not None and rope_cos_sin is not None,
               "ROPE needs positions and rope_cos_sin")
        _check(positions.dtype == torch.int64 and tuple(positions.shape) == (T,)
               and positions.is_contiguous(), "positions must be a contiguous int64 [T]")
        tdt = torch.bfloat16 if flags & TABLE_BF16 else torch.float32
        _check(rope_cos_sin.dtype == tdt and rope_cos_sin.dim() == 2
               and rope_cos_sin.shape[1] == 64 and rope_cos_sin.is_contiguous(),
               f"rope_cos_sin must be a contiguous {tdt} [max_position, 64]")
    if q_fp8:
        _check(q_scale is not None and q_scale.dtype == torch.float32 and q_scale.numel() >= 1,
               "Q_FP8 needs an fp32 q_scale")
    if kv_fp8:
        _check(kv_scale is not None and kv_scale.dtype == torch.float32 and kv_scale.numel() >= 1,
               "KV_FP8 needs an fp32 kv_scale")
    dev = q_out.device
    _check(dev.type == "cuda", "tensors must be on a GPU")
    for t in (ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin, q_scale,
              kv_scale, *(e[1] for e in extra)):
        if t is not None:
            _check(t.device == dev, "all tensors must be on the same GPU")


def _raw_stream(index: int, stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    return _current_raw_stream(index)


try:  # torch's C-level accessor for the current stream's handle (no Stream object)
    _current_raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover
    def _current_raw_stream(index):
        return torch.cuda.current_stream(index).cuda_stream


def _launch(args: tuple, flags: int, dims: Dims, index: int, stream,
            entry: str = "mla_decode_q_concat_kv_insert") -> None:
    fn = getattr(load(), entry)
    if index == torch.cuda.current_device():
        rc = fn(*args, flags, ctypes.byref(dims), _raw_stream(index, stream))
    else:
        with torch.cuda.device(index):
            rc = fn(*args, flags, ctypes.byref(dims), _raw_stream(index, stream))
    if rc != OK:
        raise MlaDqError(rc, strerror(rc))


class PreparedInsert:
    """The epilogue bound to fixed tensors: arguments are checked and
    marshalled once, and each call only enqueues the launch (for loops over
    static buffers, e.g. under stream capture).  Same arguments as
    mla_decode_q_concat_kv_insert; the tensors must stay alive and keep their
    storage."""

    def __init__(self, q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions=None,
                 rope_cos_sin=None, q_scale=None, kv_scale=None, flags: int = 0):
        tensors = (q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                   rope_cos_sin, q_scale, kv_scale)
        _validate_only(*tensors, flags)
        self._tensors = tensors
        self._args = tuple(_ptr(t) for t in tensors)
        self._dims = _dims(ql_nope, q_pe, kv_c, k_pe, cache, rope_cos_sin)
        self._flags = flags
        self._index = q_out.device.index

    def __call__(self, stream=None) -> None:
        _launch(self._args, self._flags, self._dims, self._index, stream)


def _validate_uk(q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                 rope_cos_sin, q_scale, kv_scale, flags) -> None:
    H = q_nope.shape[1] if q_nope.dim() == 3 else -1
    _check(w_uk_t.dim() == 3 and tuple(w_uk_t.shape) == (H, 512, 128) and w_uk_t.is_contiguous(),
           "w_uk_t must be a contiguous [H, 512, 128] tensor (W_UK transposed per head)")
    _validate_only(q_out, q_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions, rope_cos_sin,
                   q_scale, kv_scale, flags, "q_nope", 128, (("w_uk_t", w_uk_t),))


def mla_decode_uk_q_concat_kv_insert(q_out: torch.Tensor, q_nope: torch.Tensor, w_uk_t: torch.Tensor,
                                     q_pe: torch.Tensor, kv_c: torch.Tensor, k_pe: torch.Tensor,
                                     cache: torch.Tensor, slot_mapping: torch.Tensor,
                                     positions: torch.Tensor | None = None,
                                     rope_cos_sin: torch.Tensor | None = None,
                                     q_scale: torch.Tensor | None = None,
                                     kv_scale: torch.Tensor | None = None, flags: int = 0,
                                     stream: torch.cuda.Stream | None = None) -> None:
    """Enqueue the epilogue fused into the W_UK product: q_out [T,H,576] gets
    enc(q_nope[t,h] @ W_UK[h]) in columns 0..511 and the rotated q_pe tail;
    the cache rows are written as by mla_decode_q_concat_kv_insert.
    ``q_nope`` is [T, H, 128] (strided, e.g. a view of the q projection's
    [T, H, 192] output) and ``w_uk_t`` [H, 512, 128] holds each head's W_UK
    transposed."""
    _validate_uk(q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                 rope_cos_sin, q_scale, kv_scale, flags)
    dims = _dims(q_nope, q_pe, kv_c, k_pe, cache, rope_cos_sin)
    args = (_ptr(q_out), _ptr(q_nope), _ptr(w_uk_t), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe), _ptr(cache),
            _ptr(slot_mapping), _ptr(positions), _ptr(rope_cos_sin), _ptr(q_scale), _ptr(kv_scale))
    _launch(args, flags, dims, q_out.device.index, stream, "mla_decode_uk_q_concat_kv_insert")


class PreparedUkInsert:
    """mla_decode_uk_q_concat_kv_insert bound to fixed tensors (checked and
    marshalled once; each call only enqueues the launch)."""

    def __init__(self, q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions=None,
                 rope_cos_sin=None, q_scale=None, kv_scale=None, flags: int = 0):
        tensors = (q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                   rope_cos_sin, q_scale, kv_scale)
        _validate_uk(*tensors, flags)
        self._tensors = tensors
        self._args = tuple(_ptr(t) for t in tensors)
        self._dims = _dims(q_nope, q_pe, kv_c, k_pe, cache, rope_cos_sin)
        self._flags = flags
        self._index = q_out.device.index

    def __call__(self, stream=None) -> None:
        _launch(self._args, self._flags, self._dims, self._index, stream, "mla_decode_uk_q_concat_kv_insert")


def fused_mla_decode_q_concat_kv_cache_insert(ql_nope: torch.Tensor, q_pe: torch.Tensor,
                                              kv_c: torch.Tensor, k_pe: torch.Tensor,
                                              cache: torch.Tensor, slot_mapping: torch.Tensor,
                                              positions: torch.Tensor | None = None,
                                              rope_cos_sin: torch.Tensor | None = None,
                                              q_scale: torch.Tensor | None = None,
                                              kv_scale: torch.Tensor | None = None,
                                              q_fp8: bool = False,
                                              rope_style: str = "neox") -> torch.Tensor:
    """The page's user-level call: allocates and returns q [T, H, 576] and
    updates ``cache`` in place.  RoPE is on when positions and a table are
    given (``rope_style`` "neox" or "gptj"); fp16 activations, a bf16 table
    and an e4m3 cache follow from the tensors' dtypes."""
    T, H = ql_nope.shape[0], ql_nope.shape[1]
    flags = 0
    if positions is not None or rope_cos_sin is not None:
        flags |= ROPE
        if rope_style == "gptj":
            flags |= ROPE_GPTJ
        elif rope_style != "neox":
            raise ValueError("rope_style must be 'neox' or 'gptj'")
        if rope_cos_sin is not None and rope_cos_sin.dtype == torch.bfloat16:
            flags |= TABLE_BF16
    if ql_nope.dtype == torch.float16:
        flags |= FP16
    if q_fp8:
        flags |= Q_FP8
    if cache.dtype in _FP8:
        flags |= KV_FP8
    q = torch.empty((T, H, 576), device=ql_nope.device,
                    dtype=torch.float8_e4m3fn if q_fp8 else ql_nope.dtype)
    mla_decode_q_concat_kv_insert(q, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                                  rope_cos_sin, q_scale, kv_scale, flags)
    return q


# ---- MLA decode attention over the paged latent cache (include/mla_attn.h) ----

ATTN_Q_FP8 = 1 << 0
ATTN_KV_FP8 = 1 << 1
ERR_WORKSPACE = -7
ERR_SCRATCH = -8
SCRATCH_BYTES = 16 << 20     # MLA_ATTN_SCRATCH_BYTES: the no-alloc entry point's buffer

ATTN_EXPORTED_SYMBOLS = ("mla_decode_attention", "mla_decode_attention_workspace_size",
                         "mla_decode_attention_plan", "mla_decode_attention_noalloc")


class AttnDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "num_heads", "num_blocks", "block_size", "max_blocks_per_seq", "max_seq_len")]


class AttnPlan(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int32), ("keys_per_split", ctypes.c_int32),
                ("head_tiles", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("target_workgroups", ctypes.c_int64), ("xcd_remap", ctypes.c_int32),
                ("block_threads", ctypes.c_int32)]


def _attn_lib() -> ctypes.CDLL:
    lib = load()
    if not getattr(lib, "_attn_configured", False):
        vp = ctypes.c_void_p
        lib.mla_decode_attention.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_uint32,
            ctypes.POINTER(AttnDims), vp]
        lib.mla_decode_attention.restype = ctypes.c_int
        lib.mla_decode_attention_noalloc.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_uint32, ctypes.POINTER(AttnDims), vp]
        lib.mla_decode_attention_noalloc.restype = ctypes.c_int
        lib.mla_decode_attention_workspace_size.argtypes = [ctypes.POINTER(AttnDims),
                                                            ctypes.c_uint32]
        lib.mla_decode_attention_workspace_size.restype = ctypes.c_size_t
        lib.mla_decode_attention_plan.argtypes = [ctypes.POINTER(AttnDims), ctypes.c_uint32,
                                                  ctypes.POINTER(AttnPlan)]
        lib.mla_decode_attention_plan.restype = ctypes.c_int
        lib._attn_configured = True
    return lib


def attn_plan(dims: AttnDims, flags: int) -> AttnPlan:
    p = AttnPlan()
    rc = _attn_lib().mla_decode_attention_plan(ctypes.byref(dims), ctypes.c_uint32(flags),
                                               ctypes.byref(p))
    if rc != OK:
        raise MlaDqError(rc, strerror(rc))
    return p


def attn_workspace_size(dims: AttnDims, flags: int) -> int:
    return int(_attn_lib().mla_decode_attention_workspace_size(ctypes.byref(dims),
                                                               ctypes.c_uint32(flags)))


def _attn_flags(q: torch.Tensor, cache: torch.Tensor) -> int:
    return (ATTN_Q_FP8 if q.dtype in _FP8 else 0) | (ATTN_KV_FP8 if cache.dtype in _FP8 else 0)


def _attn_dims(q, cache, block_table, max_seq_len) -> AttnDims:
    d = AttnDims()
    d.batch, d.num_heads = q.shape[0], q.shape[1]
    d.num_blocks, d.block_size = cache.shape[0], cache.shape[1]
    d.max_blocks_per_seq = block_table.shape[1]
    d.max_seq_len = (block_table.shape[1] * cache.shape[1] if max_seq_len is None
                     else int(max_seq_len))
    return d


def _attn_validate(out, q, cache, block_table, seq_lens, q_scale, kv_scale) -> None:
    _check(q.dim() == 3 and q.shape[2] == 576 and q.is_contiguous(),
           "q must be a contiguous [B, H, 576] tensor")
    B_, H = q.shape[0], q.shape[1]
    _check(tuple(out.shape) == (B_, H, 512) and out.dtype == torch.bfloat16
           and out.is_contiguous(), "out must be a contiguous bf16 [B, H, 512] tensor")
    _check(cache.dim() == 3 and cache.shape[2] == 576 and cache.is_contiguous(),
           "cache must be a contiguous [num_blocks, block_size, 576] tensor")
    _check(q.dtype in _FP8 or q.dtype == torch.bfloat16, "q must be bf16 or e4m3")
    _check(cache.dtype in _FP8 or cache.dtype == torch.bfloat16, "cache must be bf16 or e4m3")
    _check(block_table.dtype == torch.int32 and block_table.dim() == 2
           and block_table.shape[0] == B_ and block_table.is_contiguous(),
           "block_table must be a contiguous int32 [B, max_blocks_per_seq]")
    _check(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B_,)
           and seq_lens.is_contiguous(), "seq_lens must be a contiguous int32 [B]")
    if q.dtype in _FP8:
        _check(q_scale is not None and q_scale.dtype == torch.float32, "e4m3 q needs q_scale")
    if cache.dtype in _FP8:
        _check(kv_scale is not None and kv_scale.dtype == torch.float32,
               "e4m3 cache needs kv_scale")
    dev = out.device
    _check(dev.type == "cuda", "tensors must be on a GPU")
    for t in (q, cache, block_table, seq_lens, q_scale, kv_scale):
        if t is not None:
            _check(t.device == dev, "all tensors must be on the same GPU")


class PreparedAttention:
    """Decode attention bound to fixed tensors and a workspace: checked and
    marshalled once, each call only enqueues the kernels (for loops over
    static buffers, e.g. under stream capture).  ``max_seq_len`` bounds every
    seq_lens entry (default: the block table's capacity); the key split is
    planned from it."""

    def __init__(self, out, q, cache, block_table, seq_lens, sm_scale: float, q_scale=None,
                 kv_scale=None, max_seq_len: int | None = None,
                 workspace: torch.Tensor | None = None):
        _attn_validate(out, q, cache, block_table, seq_lens, q_scale, kv_scale)
        self._dims = _attn_dims(q, cache, block_table, max_seq_len)
        self._flags = _attn_flags(q, cache)
        self.plan = attn_plan(self._dims, self._flags)
        need = int(self.plan.workspace_bytes)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=out.device)
        if need > 0:
            _check(workspace.device == out.device and workspace.is_contiguous()
                   and workspace.numel() * workspace.element_size() >= need,
                   f"workspace must be a contiguous buffer of at least {need} bytes")
        self._tensors = (out, q, cache, block_table, seq_lens, q_scale, kv_scale, workspace)
        self._args = (_ptr(out), _ptr(q), _ptr(cache), _ptr(block_table), _ptr(seq_lens),
                      _ptr(q_scale), _ptr(kv_scale))
        self._sm_scale = float(sm_scale)
        self._ws = _ptr(workspace) if need > 0 else None
        self._ws_bytes = workspace.numel() * workspace.element_size() if need > 0 else 0
        self._index = out.device.index

    def __call__(self, stream=None) -> None:
        fn = _attn_lib().mla_decode_attention
        args = (*self._args, ctypes.c_float(self._sm_scale), self._ws,
                ctypes.c_size_t(self._ws_bytes), ctypes.c_uint32(self._flags),
                ctypes.byref(self._dims))
        if self._index == torch.cuda.current_device():
            rc = fn(*args, _raw_stream(self._index, stream))
        else:
            with torch.cuda.device(self._index):
                rc = fn(*args, _raw_stream(self._index, stream))
        if rc != OK:
            raise MlaDqError(rc, strerror(rc))


def mla_decode_attention(q: torch.Tensor, cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, sm_scale: float,
                         q_scale: torch.Tensor | None = None,
                         kv_scale: torch.Tensor | None = None,
                         max_seq_len: int | None = None,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention of q [B, H, 576] over the paged latent cache; returns
    bf16 [B, H, 512].  E4M3 q or cache follow from the dtypes (with their
    fp32 scales)."""
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    PreparedAttention(out, q, cache, block_table, seq_lens, sm_scale, q_scale, kv_scale,
                      max_seq_len)()
    return out


def mla_decode_attention_noalloc(out: torch.Tensor, q: torch.Tensor, cache: torch.Tensor,
                                 block_table: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
                                 q_scale: torch.Tensor | None = None,
                                 kv_scale: torch.Tensor | None = None,
                                 max_seq_len: int | None = None, stream=None) -> torch.Tensor:
    """Decode attention into the caller's ``out`` through the entry point that
    allocates nothing (include/mla_attn.h): split ranges use the library's
    per-GPU scratch buffer, so calls on one GPU must be ordered.  Raises
    MlaDqError (code ERR_SCRATCH) if the split needs more than SCRATCH_BYTES."""
    _attn_validate(out, q, cache, block_table, seq_lens, q_scale, kv_scale)
    d = _attn_dims(q, cache, block_table, max_seq_len)
    args = (_ptr(out), _ptr(q), _ptr(cache), _ptr(block_table), _ptr(seq_lens), _ptr(q_scale),
            _ptr(kv_scale), ctypes.c_float(float(sm_scale)), ctypes.c_uint32(_attn_flags(q, cache)),
            ctypes.byref(d))
    fn = _attn_lib().mla_decode_attention_noalloc
    index = out.device.index
    if index == torch.cuda.current_device():
        rc = fn(*args, _raw_stream(index, stream))
    else:
        with torch.cuda.device(index):
            rc = fn(*args, _raw_stream(index, stream))
    if rc != OK:
        raise MlaDqError(rc, strerror(rc))
    return out
