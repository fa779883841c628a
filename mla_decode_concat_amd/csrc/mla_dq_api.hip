// C ABI of the fused MLA decode epilogue: argument validation, the choice of
// mapping, and the launch on the caller's stream.  The contract is in
// include/mla_dq.h.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>
#include <stdlib.h>

#include "mla_attn.h"
#include "mla_dq.h"
#include "mla_dq_internal.h"

namespace mla_dq {
namespace {

constexpr int kNothingToDo = 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) touched by a strided bf16 tensor [T, H, width].
struct Extent {
    uintptr_t lo, hi;
};

Extent extent3(const void* p, int64_t T, int64_t H, int64_t st, int64_t sh, int64_t width,
               int64_t elem_bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    const int64_t last = (T - 1) * st + (H - 1) * sh + width;
    return Extent{b, b + uintptr_t(last) * uintptr_t(elem_bytes)};
}

Extent span(const void* p, int64_t bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Extent{b, b + uintptr_t(bytes)};
}

// An empty extent (lo == hi) overlaps nothing.
bool overlap(Extent x, Extent y) { return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi; }

int64_t env_int64(const char* name, int64_t fallback) {
    const char* s = getenv(name);
    if (s == nullptr || *s == '\0') return fallback;
    char* end = nullptr;
    const long long n = strtoll(s, &end, 10);
    if (end == s || *end != '\0' || n < 0) return fallback;
    return int64_t(n);
}

// The environment variable, when set, applies to every head count.
int64_t small_rows_max(int64_t H) {
    static const int64_t v = env_int64("MLA_DQ_SMALL_ROWS_MAX", -1);
    if (v >= 0) return v;
    return H <= kFewHeadsMax ? kDefaultSmallRowsMaxFewHeads : kDefaultSmallRowsMax;
}

int64_t mid_rows_max() {
    static const int64_t v = env_int64("MLA_DQ_MID_ROWS_MAX", kDefaultMidRowsMax);
    return v;
}

int64_t stream_bytes_min() {
    static const int64_t v = env_int64("MLA_DQ_STREAM_BYTES_MIN", kDefaultStreamBytesMin);
    return v;
}

// Bytes one call reads and writes: each 576-wide input row once (2-byte
// elements), each output row once, plus slot, position and rope table row
// per token.  A launch restricted to one kind of row counts only its rows
// (and the slot only with the cache row).
int64_t call_bytes(const mla_dq_dims* d, uint32_t flags) {
    const int64_t T = d->num_tokens, H = d->num_heads;
    const bool rope = flags & MLA_DQ_ROPE;
    const int64_t qh = (flags & MLA_DQ_CACHE_ROWS_ONLY) ? 0 : H;     // query rows per token
    const int64_t kv = (flags & MLA_DQ_Q_ROWS_ONLY) ? 0 : 1;         // cache rows per token
    const int64_t table_row = (flags & MLA_DQ_TABLE_BF16) ? 128 : 256;
    const int64_t read = T * (qh * 1152 + kv * (1152 + 8) + (rope ? 8 + table_row : 0));
    const int64_t write = T * 576 * (qh * ((flags & MLA_DQ_Q_FP8) ? 1 : 2) +
                                     kv * ((flags & MLA_DQ_KV_FP8) ? 1 : 2));
    return read + write;
}

int64_t uk_large_rows_min() {
    static const int64_t v = env_int64("MLA_DQ_UK_LARGE_ROWS_MIN", kDefaultUkLargeRowsMin);
    return v;
}

// Bytes of the fused product's call: q_nope (128 elements per query row)
// instead of ql_nope, W_UK once, and the rest of the epilogue's traffic.
int64_t uk_call_bytes(const mla_dq_dims* d, uint32_t flags) {
    const int64_t T = d->num_tokens, H = d->num_heads;
    const bool rope = flags & MLA_DQ_ROPE;
    const int64_t table_row = (flags & MLA_DQ_TABLE_BF16) ? 128 : 256;
    const int64_t read = T * H * (256 + 128) + H * 512 * 128 * 2 +
                         T * (1152 + 8 + (rope ? 8 + table_row : 0));
    const int64_t write = T * 576 * (H * ((flags & MLA_DQ_Q_FP8) ? 1 : 2) + ((flags & MLA_DQ_KV_FP8) ? 1 : 2));
    return read + write;
}

constexpr uint32_t kUkOnlyUnsupported = MLA_DQ_Q_ROWS_ONLY | MLA_DQ_CACHE_ROWS_ONLY | MLA_DQ_FORCE_MID_T;

// Checks that do not need any pointer: flags and shapes.
int check_flags_dims(uint32_t flags, const mla_dq_dims* d) {
    if (d == nullptr) return MLA_DQ_ERR_NULL;
    const uint32_t known = MLA_DQ_ROPE | MLA_DQ_Q_FP8 | MLA_DQ_KV_FP8 | MLA_DQ_FP16 |
                           MLA_DQ_ROPE_GPTJ | MLA_DQ_TABLE_BF16 | MLA_DQ_FORCE_SMALL_T |
                           MLA_DQ_FORCE_LARGE_T | MLA_DQ_FORCE_STREAM | MLA_DQ_FORCE_CACHED |
                           MLA_DQ_FORCE_MID_T | MLA_DQ_Q_ROWS_ONLY | MLA_DQ_CACHE_ROWS_ONLY;
    if (flags & ~known) return MLA_DQ_ERR_FLAGS;
    if ((flags & MLA_DQ_Q_ROWS_ONLY) && (flags & MLA_DQ_CACHE_ROWS_ONLY)) return MLA_DQ_ERR_FLAGS;
    if ((flags & (MLA_DQ_ROPE_GPTJ | MLA_DQ_TABLE_BF16)) && !(flags & MLA_DQ_ROPE))
        return MLA_DQ_ERR_FLAGS;
    const uint32_t forced_mappings = flags & (MLA_DQ_FORCE_SMALL_T | MLA_DQ_FORCE_MID_T | MLA_DQ_FORCE_LARGE_T);
    if (forced_mappings & (forced_mappings - 1)) return MLA_DQ_ERR_FLAGS;   // more than one
    if ((flags & MLA_DQ_FORCE_STREAM) && (flags & MLA_DQ_FORCE_CACHED)) return MLA_DQ_ERR_FLAGS;
    const int64_t T = d->num_tokens, H = d->num_heads;
    if (T < 0 || H < 1 || d->num_blocks < 1 || d->block_size < 1) return MLA_DQ_ERR_DIM;
    // Row indices, and T * (H + 1) * 72 chunk counts, stay below 2^31.
    if (H > INT32_MAX / kRowChunks - 1) return MLA_DQ_ERR_DIM;
    if (T > INT32_MAX / (kRowChunks * (H + 1))) return MLA_DQ_ERR_DIM;
    if (d->num_blocks > (INT64_MAX / 2048) / d->block_size) return MLA_DQ_ERR_DIM;
    if (flags & MLA_DQ_ROPE) {
        if (d->max_position < 1 || d->max_position > (int64_t(1) << 40)) return MLA_DQ_ERR_DIM;
    }
    const int64_t strides[] = {d->ql_nope_stride_t, d->ql_nope_stride_h, d->q_pe_stride_t,
                               d->q_pe_stride_h, d->kv_c_stride_t, d->k_pe_stride_t};
    for (int64_t s : strides)
        if (s < 0 || s > (int64_t(1) << 40)) return MLA_DQ_ERR_DIM;
    if (T == 0) return kNothingToDo;
    // Row strides must keep every 16-byte chunk aligned; a stride that is
    // never used (one token, one head) may be anything.
    const bool many_t = T > 1, many_h = H > 1;
    if ((many_t && (d->ql_nope_stride_t % 8 || d->q_pe_stride_t % 8 || d->kv_c_stride_t % 8 ||
                    d->k_pe_stride_t % 8)) ||
        (many_h && (d->ql_nope_stride_h % 8 || d->q_pe_stride_h % 8)))
        return MLA_DQ_ERR_ALIGN;
    return MLA_DQ_OK;
}

}  // namespace

// Rows per token of a launch: all H + 1, or only the H query rows, or only
// the cache row.
int64_t row_stride(int64_t H, uint32_t flags) {
    if (flags & MLA_DQ_Q_ROWS_ONLY) return H;
    if (flags & MLA_DQ_CACHE_ROWS_ONLY) return 1;
    return H + 1;
}

int plan(const mla_dq_dims* d, uint32_t flags, mla_dq_launch_plan* out) {
    if (out == nullptr) return MLA_DQ_ERR_NULL;
    const int rc = check_flags_dims(flags, d);
    if (rc < 0) return rc;
    const int64_t T = d->num_tokens, H = d->num_heads;
    const int64_t rows = T * row_stride(H, flags);
    const int64_t rows_thr = small_rows_max(H), mid_thr = mid_rows_max(), bytes_thr = stream_bytes_min();
    const int64_t bytes = call_bytes(d, flags);
    int mapping = rows <= rows_thr ? 0 : (rows <= mid_thr ? 2 : 1);
    if (flags & MLA_DQ_FORCE_SMALL_T) mapping = 0;
    if (flags & MLA_DQ_FORCE_MID_T) mapping = 2;
    if (flags & MLA_DQ_FORCE_LARGE_T) mapping = 1;
    int streaming = bytes >= bytes_thr ? 1 : 0;
    if (flags & MLA_DQ_FORCE_STREAM) streaming = 1;
    if (flags & MLA_DQ_FORCE_CACHED) streaming = 0;
    const Mapping& m = mapping == 0 ? kSmallMapping : (mapping == 2 ? kMidMapping : kLargeMapping);
    int rows_per_wave = m.rows_per_wave;
    if (mapping == 1 && !streaming && bytes >= kMidSizeBytesMin && bytes <= kMidSizeBytesMax)
        rows_per_wave = kMidSizeRowsPerWave;
    const int64_t latent_per_block = int64_t(m.block / 64) * rows_per_wave;
    const int64_t tails_per_block = int64_t(m.block / 8) * m.tail_steps;
    int64_t tail_blocks = (rows + tails_per_block - 1) / tails_per_block;
#if MLA_DQ_XCD_REMAP
    // A multiple of 8 keeps every latent workgroup on the XCD its index
    // implies (workgroups are dealt to the 8 XCDs round-robin).
    tail_blocks = (tail_blocks + 7) / 8 * 8;
#endif
    out->mapping = mapping;
    out->streaming = streaming;
    out->block_threads = m.block;
    out->rows_per_wave = rows_per_wave;
    out->tail_steps = m.tail_steps;
    out->reserved = 0;
    out->small_rows_max = rows_thr;
    out->stream_bytes_min = bytes_thr;
    out->bytes = bytes;
    out->tail_blocks = T == 0 ? 0 : tail_blocks;
    out->latent_blocks = (rows + latent_per_block - 1) / latent_per_block;
    out->grid_blocks = out->tail_blocks + out->latent_blocks;
    out->total_rows = rows;
    out->mid_rows_max = mid_thr;
    return MLA_DQ_OK;
}

namespace {

// Pointer checks of both entry points.  `nope` is ql_nope [T, H, 512] or, for
// the fused product, q_nope [T, H, 128] (nope_width elements per row, the
// ql_nope strides of dims); `extra` is one more input extent (W_UK) or empty.
int validate_io(void* q_out, const void* nope, int64_t nope_width, Extent extra, const void* q_pe,
                const void* kv_c, const void* k_pe, void* cache, const int64_t* slot_mapping,
                const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
                const float* kv_scale, uint32_t flags, const mla_dq_dims* d) {
    const void* ql_nope = nope;
    const bool rope = flags & MLA_DQ_ROPE, qf8 = flags & MLA_DQ_Q_FP8, kvf8 = flags & MLA_DQ_KV_FP8;
    if (!q_out || !ql_nope || !q_pe || !kv_c || !k_pe || !cache || !slot_mapping)
        return MLA_DQ_ERR_NULL;
    if (rope && (!positions || !rope_cos_sin)) return MLA_DQ_ERR_NULL;
    if ((qf8 && !q_scale) || (kvf8 && !kv_scale)) return MLA_DQ_ERR_NULL;
    if (!aligned(q_out, 16) || !aligned(ql_nope, 16) || !aligned(q_pe, 16) || !aligned(kv_c, 16) ||
        !aligned(k_pe, 16) || !aligned(cache, 16) || !aligned(slot_mapping, 8))
        return MLA_DQ_ERR_ALIGN;
    if (rope && (!aligned(positions, 8) || !aligned(rope_cos_sin, 16))) return MLA_DQ_ERR_ALIGN;
    if ((qf8 && !aligned(q_scale, 4)) || (kvf8 && !aligned(kv_scale, 4))) return MLA_DQ_ERR_ALIGN;

    const int64_t T = d->num_tokens, H = d->num_heads;
    const int64_t slots = d->num_blocks * d->block_size;
    const Extent q{reinterpret_cast<uintptr_t>(q_out),
                   reinterpret_cast<uintptr_t>(q_out) + uintptr_t(T * H * 576 * (qf8 ? 1 : 2))};
    const Extent c{reinterpret_cast<uintptr_t>(cache),
                   reinterpret_cast<uintptr_t>(cache) + uintptr_t(slots * 576 * (kvf8 ? 1 : 2))};
    // Every input the flags make the kernel read: some workgroups may read
    // one after others have stored rows, so no output may overlap any of them.
    const Extent none{0, 0};
    const int64_t table_row = (flags & MLA_DQ_TABLE_BF16) ? 128 : 256;
    const Extent in[] = {
        extent3(ql_nope, T, H, d->ql_nope_stride_t, d->ql_nope_stride_h, nope_width, 2),
        extra,
        extent3(q_pe, T, H, d->q_pe_stride_t, d->q_pe_stride_h, 64, 2),
        extent3(kv_c, T, 1, d->kv_c_stride_t, 0, 512, 2),
        extent3(k_pe, T, 1, d->k_pe_stride_t, 0, 64, 2),
        span(slot_mapping, T * 8),
        rope ? span(positions, T * 8) : none,
        rope ? span(rope_cos_sin, d->max_position * table_row) : none,
        qf8 ? span(q_scale, 4) : none,
        kvf8 ? span(kv_scale, 4) : none,
    };
    if (overlap(q, c)) return MLA_DQ_ERR_ALIAS;
    for (const Extent& e : in)
        if (overlap(q, e) || overlap(c, e)) return MLA_DQ_ERR_ALIAS;
    return MLA_DQ_OK;
}

// The fields both launches share; the row enumeration (row_stride,
// first_head, rows_per_token, total_rows, tail_blocks) is the caller's.
KernelArgs common_args(void* q_out, const void* nope, const void* q_pe, const void* kv_c,
                       const void* k_pe, void* cache, const int64_t* slot_mapping,
                       const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
                       const float* kv_scale, uint32_t flags, const mla_dq_dims* dims) {
    KernelArgs a;
    a.q_out = static_cast<uint8_t*>(q_out);
    a.ql_nope = static_cast<const uint16_t*>(nope);
    a.q_pe = static_cast<const uint16_t*>(q_pe);
    a.kv_c = static_cast<const uint16_t*>(kv_c);
    a.k_pe = static_cast<const uint16_t*>(k_pe);
    a.cache = static_cast<uint8_t*>(cache);
    a.slot_mapping = slot_mapping;
    a.positions = positions;
    a.rope_cos_sin = rope_cos_sin;
    a.q_scale = q_scale;
    a.kv_scale = kv_scale;
    a.ql_nope_st = dims->ql_nope_stride_t;
    a.ql_nope_sh = dims->ql_nope_stride_h;
    a.q_pe_st = dims->q_pe_stride_t;
    a.q_pe_sh = dims->q_pe_stride_h;
    a.kv_c_st = dims->kv_c_stride_t;
    a.k_pe_st = dims->k_pe_stride_t;
    a.num_slots = dims->num_blocks * dims->block_size;
    a.max_position = (flags & MLA_DQ_ROPE) ? dims->max_position : 1;
    a.num_heads = uint32_t(dims->num_heads);
    a.fp16 = (flags & MLA_DQ_FP16) ? 1u : 0u;
    a.gptj = (flags & MLA_DQ_ROPE_GPTJ) ? 1u : 0u;
    a.table_bf16 = (flags & MLA_DQ_TABLE_BF16) ? 1u : 0u;
    return a;
}

}  // namespace

int validate(void* q_out, const void* ql_nope, const void* q_pe, const void* kv_c,
             const void* k_pe, void* cache, const int64_t* slot_mapping,
             const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
             const float* kv_scale, uint32_t flags, const mla_dq_dims* d) {
    const int rc = check_flags_dims(flags, d);
    if (rc != MLA_DQ_OK) return rc;
    return validate_io(q_out, ql_nope, 512, Extent{0, 0}, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                       rope_cos_sin, q_scale, kv_scale, flags, d);
}

int uk_validate(void* q_out, const void* q_nope, const void* w_uk_t, const void* q_pe,
                const void* kv_c, const void* k_pe, void* cache, const int64_t* slot_mapping,
                const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
                const float* kv_scale, uint32_t flags, const mla_dq_dims* d) {
    if (flags & kUkOnlyUnsupported) return MLA_DQ_ERR_FLAGS;
    const int rc = check_flags_dims(flags, d);
    if (rc != MLA_DQ_OK) return rc;
    if (!w_uk_t) return MLA_DQ_ERR_NULL;
    if (!aligned(w_uk_t, 16)) return MLA_DQ_ERR_ALIGN;
    return validate_io(q_out, q_nope, 128, span(w_uk_t, d->num_heads * 512 * 128 * 2), q_pe, kv_c, k_pe,
                       cache, slot_mapping, positions, rope_cos_sin, q_scale, kv_scale, flags, d);
}

int uk_plan(const mla_dq_dims* d, uint32_t flags, mla_dq_uk_launch_plan* out) {
    if (out == nullptr) return MLA_DQ_ERR_NULL;
    if (flags & kUkOnlyUnsupported) return MLA_DQ_ERR_FLAGS;
    const int rc = check_flags_dims(flags, d);
    if (rc < 0) return rc;
    const int64_t T = d->num_tokens, H = d->num_heads;
    const int64_t large_min = uk_large_rows_min(), bytes_thr = stream_bytes_min();
    const int64_t bytes = uk_call_bytes(d, flags);
    int mapping = T * H >= large_min ? 1 : 0;
    if (flags & MLA_DQ_FORCE_SMALL_T) mapping = 0;
    if (flags & MLA_DQ_FORCE_LARGE_T) mapping = 1;
    int streaming = bytes >= bytes_thr ? 1 : 0;
    if (flags & MLA_DQ_FORCE_STREAM) streaming = 1;
    if (flags & MLA_DQ_FORCE_CACHED) streaming = 0;
    const int64_t block = MLA_DQ_UK_BLOCK, waves = block / 64;
    const int64_t tail_steps = mapping ? kLargeMapping.tail_steps : 1;
    int64_t nb = mapping ? MLA_DQ_UK_LARGE_NB : MLA_DQ_UK_SMALL_NB;
    if (mapping && T * H <= MLA_DQ_UK_LARGE_NB2_ROWS_MAX && T >= MLA_DQ_UK_LARGE_NB2_TOKENS_MIN) nb = 2;
    int64_t groups = 512 / (waves * 16 * nb);
    int64_t tpg = mapping ? MLA_DQ_UK_LARGE_TOKENS : MLA_DQ_UK_SMALL_TOKENS;
    const int64_t target = mapping ? MLA_DQ_UK_TARGET_BLOCKS : MLA_DQ_UK_SMALL_TARGET_BLOCKS;
    while (tpg > 16 && H * ((T + tpg - 1) / tpg) * groups < target) tpg /= 2;
    if (!mapping && H * ((T + tpg - 1) / tpg) <= MLA_DQ_UK_SMALL_NB1_UNITS_MAX) {
        nb = 1;
        groups = 512 / (waves * 16);
    }
    const int64_t units = H * ((T + tpg - 1) / tpg);
    const int64_t product_blocks = 8 * groups * ((units + 7) / 8);   // 8 XCDs x ceil(units / 8) units
    const int64_t tails_per_block = (block / 8) * tail_steps;
    const int64_t tail_blocks = (T * (H + 1) + tails_per_block - 1) / tails_per_block;
    const int64_t cache_blocks = (T + waves - 1) / waves;
    const int64_t grid = product_blocks + tail_blocks + cache_blocks;
    // Work-item indices of a launch stay below 2^32.
    if (grid * block > int64_t(UINT32_MAX)) return MLA_DQ_ERR_DIM;
    out->mapping = mapping;
    out->streaming = streaming;
    out->block_threads = int32_t(block);
    out->n_blocks = int32_t(nb);
    out->tail_steps = int32_t(tail_steps);
    out->tokens_per_group = int32_t(tpg);
    out->head_major = H >= MLA_DQ_UK_HEAD_MAJOR_HEADS_MIN ? 1 : 0;
    out->reserved = 0;
    out->column_groups = groups;
    out->units = units;
    out->product_blocks = product_blocks;
    out->tail_blocks = tail_blocks;
    out->cache_blocks = cache_blocks;
    out->grid_blocks = grid;
    out->bytes = bytes;
    out->flops = 2 * T * H * 128 * 512;
    out->stream_bytes_min = bytes_thr;
    out->large_rows_min = large_min;
    return MLA_DQ_OK;
}

}  // namespace mla_dq

extern "C" {

int mla_decode_q_concat_kv_insert(void* q_out, const void* ql_nope, const void* q_pe,
                                  const void* kv_c, const void* k_pe, void* cache,
                                  const int64_t* slot_mapping, const int64_t* positions,
                                  const float* rope_cos_sin, const float* q_scale,
                                  const float* kv_scale, uint32_t flags,
                                  const mla_dq_dims* dims, void* stream) {
    int rc = mla_dq::validate(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                              rope_cos_sin, q_scale, kv_scale, flags, dims);
    if (rc == mla_dq::kNothingToDo) return MLA_DQ_OK;
    if (rc != MLA_DQ_OK) return rc;
    mla_dq_launch_plan p;
    rc = mla_dq::plan(dims, flags, &p);
    if (rc != MLA_DQ_OK) return rc;

    mla_dq::KernelArgs a = mla_dq::common_args(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slot_mapping,
                                               positions, rope_cos_sin, q_scale, kv_scale, flags, dims);
    a.row_stride = uint32_t(mla_dq::row_stride(dims->num_heads, flags));
    a.first_head = (flags & MLA_DQ_CACHE_ROWS_ONLY) ? uint32_t(dims->num_heads) : 0u;
    a.rows_per_token = make_fastdiv31(a.row_stride);
    a.total_rows = uint32_t(p.total_rows);
    a.tail_blocks = uint32_t(p.tail_blocks);
    const hipError_t e = mla_dq::launch(a, p, flags, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_DQ_OK : MLA_DQ_ERR_LAUNCH;
}

int mla_dq_plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_launch_plan* plan) {
    return mla_dq::plan(dims, flags, plan);
}

int mla_decode_uk_q_concat_kv_insert(void* q_out, const void* q_nope, const void* w_uk_t,
                                     const void* q_pe, const void* kv_c, const void* k_pe,
                                     void* cache, const int64_t* slot_mapping,
                                     const int64_t* positions, const float* rope_cos_sin,
                                     const float* q_scale, const float* kv_scale, uint32_t flags,
                                     const mla_dq_dims* dims, void* stream) {
    int rc = mla_dq::uk_validate(q_out, q_nope, w_uk_t, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                                 rope_cos_sin, q_scale, kv_scale, flags, dims);
    if (rc == mla_dq::kNothingToDo) return MLA_DQ_OK;
    if (rc != MLA_DQ_OK) return rc;
    mla_dq_uk_launch_plan p;
    rc = mla_dq::uk_plan(dims, flags, &p);
    if (rc != MLA_DQ_OK) return rc;

    const int64_t T = dims->num_tokens, H = dims->num_heads;
    mla_dq::UkArgs u;
    u.tails = mla_dq::common_args(q_out, q_nope, q_pe, kv_c, k_pe, cache, slot_mapping, positions,
                                  rope_cos_sin, q_scale, kv_scale, flags, dims);
    u.tails.row_stride = uint32_t(H + 1);
    u.tails.first_head = 0u;
    u.tails.rows_per_token = make_fastdiv31(u.tails.row_stride);
    u.tails.total_rows = uint32_t(T * (H + 1));
    u.tails.tail_blocks = uint32_t(p.tail_blocks);
    u.cache_rows = u.tails;
    u.cache_rows.row_stride = 1u;
    u.cache_rows.first_head = uint32_t(H);
    u.cache_rows.rows_per_token = make_fastdiv31(1u);
    u.cache_rows.total_rows = uint32_t(T);
    u.cache_rows.tail_blocks = 0u;
    u.q_nope = static_cast<const uint16_t*>(q_nope);
    u.w_uk_t = static_cast<const uint16_t*>(w_uk_t);
    u.q_nope_st = dims->ql_nope_stride_t;
    u.q_nope_sh = dims->ql_nope_stride_h;
    u.heads = make_fastdiv31(uint32_t(H));
    u.ranges = make_fastdiv31(uint32_t((T + p.tokens_per_group - 1) / p.tokens_per_group));
    u.units_per_xcd = uint32_t((p.units + 7) / 8);
    u.head_major = p.head_major;
    u.num_tokens = uint32_t(T);
    u.tokens_per_group = uint32_t(p.tokens_per_group);
    u.units = uint32_t(p.units);
    u.column_groups = uint32_t(p.column_groups);
    u.product_blocks = uint32_t(p.product_blocks);
    u.tail_blocks = uint32_t(p.tail_blocks);
    u.cache_blocks = uint32_t(p.cache_blocks);
    const hipError_t e = mla_dq::launch_uk(u, p, flags, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_DQ_OK : MLA_DQ_ERR_LAUNCH;
}

int mla_dq_uk_plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_uk_launch_plan* plan) {
    return mla_dq::uk_plan(dims, flags, plan);
}

#ifndef MLA_DQ_SOURCE_DIGEST
#define MLA_DQ_SOURCE_DIGEST "unknown"
#endif

const char* mla_dq_source_digest(void) { return MLA_DQ_SOURCE_DIGEST; }

const char* mla_dq_strerror(int code) {
    switch (code) {
        case MLA_DQ_OK: return "success";
        case MLA_DQ_ERR_NULL: return "a required pointer is NULL";
        case MLA_DQ_ERR_ALIGN: return "pointer or stride misaligned (16-byte rows, 8-element strides)";
        case MLA_DQ_ERR_DIM: return "dimension or stride out of range";
        case MLA_DQ_ERR_FLAGS: return "unknown flag bit or contradictory launch overrides";
        case MLA_DQ_ERR_LAUNCH: return "HIP kernel launch failed";
        case MLA_DQ_ERR_ALIAS: return "q_out or the cache overlaps an input, or q_out overlaps the cache";
        case MLA_ATTN_ERR_WORKSPACE: return "workspace smaller than mla_decode_attention_workspace_size()";
        case MLA_ATTN_ERR_SCRATCH:
            return "the key split needs more than the library's scratch buffer (MLA_ATTN_SCRATCH_BYTES)";
        default: return "unknown mla_dq error code";
    }
}

}  // extern "C"
