// MLA decode attention over the paged latent cache for gfx950 (MI355X).
//
// The definition is in include/mla_attn.h.  Split-KV decoding: a workgroup of
// four wavefronts handles one (sequence, tile of 16 heads, range of keys) and
// walks the range 64 keys at a time.
//
//  * Scores on the matrix cores, transposed: wave w takes keys 16w .. 16w+15
//    of the step and forms S^T[key][head] = K Q^T with v_mfma_f32_16x16x32_bf16
//    over 18 steps of 32 of the 576 dimensions.  Lane l (c = l % 16,
//    g = l / 16) loads 16 bytes of key c at dimensions 32s + 8g (operand A)
//    and holds head c's query at the same dimensions (operand B, loaded once);
//    the result leaves lane l with head c's scores for keys 4g .. 4g+3.
//  * The value part (first 512 elements) of the 64 key rows goes to LDS in
//    the cache's own row-major layout, and the scores to a small LDS table
//    indexed by lane: every wave then holds, in the same lane, head c's scores
//    for keys {16w' + 4g + i}, i.e. all 64 keys between the four lanes
//    c, c+16, c+32, c+48.  Each wave runs the same online softmax (base 2)
//    on them, so the running max and sum agree across the wavefronts.
//  * Values on the matrix cores: wave w owns value dimensions 128w .. 128w+127
//    and accumulates O^T[dim][head] += V^T P^T with v_mfma_f32_16x16x32_bf16,
//    32 keys per instruction.  The K index of that product is ordered so that
//    the B operand (P^T) is the lane's own probabilities as they are, and the
//    A operand (V^T) comes from two ds_read_b64_tr_b16 of the row-major value
//    tile: in each 16-lane group, lane i reads four values of row 4g + i/4 at
//    columns 4(i % 4), and the load hands lane j the four rows of column j.
//
// E4M3 operands convert exactly to bf16 (3 mantissa bits); their scales are
// applied in fp32 to the scores and to the result.  With one range per
// sequence the workgroup writes the bf16 output itself; otherwise it writes
// (max, sum, unnormalised output) to the workspace and a second kernel merges
// the ranges.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include "mla_attn.h"
#include "mla_dq.h"

namespace mla_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRow = 576;           // latent row: 512 value + 64 positional elements
constexpr int kValue = 512;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepKeys = 16 * kWaves;   // keys per loop step
constexpr int kSteps = kRow / 32;        // 18 score products of 32 dimensions
constexpr int kVSteps = kValue / 32;     // 16 of them cover the value part
constexpr int kDimsPerWave = kValue / kWaves;
constexpr int kDimTiles = kDimsPerWave / 16;
// bf16 elements per LDS row of the value tile: 512 + 16 of padding puts the
// four rows a 16-lane group reads in one transpose load on disjoint banks.
constexpr int kVStride = kValue + 16;
constexpr int kTargetWorkgroupsDefault = 512;  // two resident workgroups per CU

struct Args {
    uint16_t* out;
    const uint8_t* q;
    const uint8_t* cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* q_scale;
    const float* kv_scale;
    float* part_o;
    float* part_m;
    float* part_l;
    float score_scale;   // sm_scale * log2(e)
    int32_t B, H, num_blocks, block_size, max_blocks, max_seq_len;
    int32_t splits, keys_per_split, head_tiles, xcd_remap;
};

// Eight E4M3 codes -> eight bf16 (exact: E4M3 values fit bf16).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 raw) {
    bf16x8 r;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], true);
        r[4 * w + 0] = (__bf16)lo.x;
        r[4 * w + 1] = (__bf16)lo.y;
        r[4 * w + 2] = (__bf16)hi.x;
        r[4 * w + 3] = (__bf16)hi.y;
    }
    return r;
}

// Raw bytes of eight consecutive elements (16 B of bf16 or 8 B of E4M3).
template <bool FP8>
struct Chunk {
    u32x4 v;
};
template <>
struct Chunk<true> {
    u32x2 v;
};

template <bool FP8>
__device__ __forceinline__ Chunk<FP8> load_chunk(const uint8_t* row, int dim) {
    Chunk<FP8> c;
    if constexpr (FP8)
        c.v = *reinterpret_cast<const u32x2*>(row + dim);
    else
        c.v = *reinterpret_cast<const u32x4*>(row + 2 * dim);
    return c;
}

template <bool FP8>
__device__ __forceinline__ bf16x8 to_bf16(Chunk<FP8> c) {
    if constexpr (FP8)
        return e4m3x8_to_bf16(c.v);
    else
        return __builtin_bit_cast(bf16x8, c.v);
}

__device__ __forceinline__ float xor_lanes(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ bf16x4 read_tr(const __bf16* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Workgroup index -> (sequence, key range, head tile).  With more than one
// head tile, the workgroups that read the same keys get consecutive logical
// indices, and the remap places consecutive logical indices on one XCD
// (workgroups are dealt to the eight XCDs in turn) so they share its L2.
__device__ __forceinline__ void decode_wg(const Args& a, int& b, int& split, int& ht) {
    int x = blockIdx.x;
    if (a.xcd_remap) {
        const int n = gridDim.x;             // a multiple of 8 when remapping
        x = (x % 8) * (n / 8) + x / 8;
    }
    ht = x % a.head_tiles;
    const int rest = x / a.head_tiles;
    split = rest % a.splits;
    b = rest / a.splits;
}

template <bool QF8, bool KVF8, bool DIRECT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_attn_partial_kernel(const Args a) {
    __shared__ __attribute__((aligned(16))) __bf16 vtile[kStepKeys * kVStride];
    __shared__ f32x4 sbuf[kWaves * 64];

    int b, split, ht;
    decode_wg(a, b, split, ht);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int k0 = split * a.keys_per_split;
    const int k1 = (k0 + a.keys_per_split < L) ? k0 + a.keys_per_split : L;
    const int head = ht * 16 + c;
    const bool head_ok = head < a.H;
    const int dim0 = w * kDimsPerWave;

    if (k0 >= k1) {
        if constexpr (DIRECT) {
            if (head_ok) {
                uint16_t* o = a.out + ((size_t)b * a.H + head) * kValue + dim0;
#pragma unroll
                for (int dt = 0; dt < kDimTiles; ++dt)
                    *reinterpret_cast<u32x2*>(o + 16 * dt + 4 * g) = u32x2{0u, 0u};
            }
        } else if (head_ok && w == 0 && g == 0) {
            const size_t p = ((size_t)b * a.H + head) * a.splits + split;
            a.part_m[p] = -INFINITY;
            a.part_l[p] = 0.0f;
        }
        return;
    }

    // Head c's query at dimensions 32s + 8g .. +7 (zero for heads past H).
    const uint8_t* qrow = a.q + ((size_t)b * a.H + (head_ok ? head : 0)) * kRow * (QF8 ? 1 : 2);
    bf16x8 qv[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        qv[s] = to_bf16<QF8>(load_chunk<QF8>(qrow, 32 * s + 8 * g));
        if (!head_ok) qv[s] = bf16x8{};
    }
    float sc = a.score_scale;
    if constexpr (QF8) sc *= *a.q_scale;
    if constexpr (KVF8) sc *= *a.kv_scale;

    const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
    const size_t row_bytes = (size_t)kRow * (KVF8 ? 1 : 2);
    auto key_row = [&](int it0) -> const uint8_t* {
        // Key c of this wave's 16 (past the range: the range's first key, masked).
        int key = it0 + 16 * w + c;
        key = key < k1 ? key : k0;
        int page = bt[key / a.block_size];
        page = page < 0 ? 0 : (page >= a.num_blocks ? a.num_blocks - 1 : page);
        return a.cache + ((size_t)page * a.block_size + key % a.block_size) * row_bytes;
    };

    Chunk<KVF8> kc[kSteps];
    {
        const uint8_t* krow = key_row(k0);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) kc[s] = load_chunk<KVF8>(krow, 32 * s + 8 * g);
    }

    f32x4 o[kDimTiles];
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.0f;
    __bf16* vrow = vtile + (16 * w + c) * kVStride;

    for (int it0 = k0; it0 < k1; it0 += kStepKeys) {
        // Every wave is done reading the previous step's tiles.
        __syncthreads();
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const bf16x8 kb = to_bf16<KVF8>(kc[s]);
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qv[s], sacc, 0, 0, 0);
            if (s < kVSteps) *reinterpret_cast<bf16x8*>(vrow + 32 * s + 8 * g) = kb;
        }
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sv[i] = (it0 + 16 * w + 4 * g + i < k1) ? sacc[i] * sc : -INFINITY;
        sbuf[w * 64 + lane] = sv;

        // The next step's keys stream in while this one finishes.
        if (it0 + kStepKeys < k1) {
            const uint8_t* krow = key_row(it0 + kStepKeys);
#pragma unroll
            for (int s = 0; s < kSteps; ++s) kc[s] = load_chunk<KVF8>(krow, 32 * s + 8 * g);
        }
        __syncthreads();

        // Head c's scores for keys 16w' + 4g + i, w' = 0..3.
        f32x4 st[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) st[v] = sbuf[v * 64 + lane];
        float bm = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v)
            bm = fmaxf(bm, fmaxf(fmaxf(st[v][0], st[v][1]), fmaxf(st[v][2], st[v][3])));
        bm = fmaxf(bm, xor_lanes(bm, 16));
        bm = fmaxf(bm, xor_lanes(bm, 32));
        const float mn = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float ps = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(st[v][i] - mn);
                ps += p;
                pb[v >> 1][4 * (v & 1) + i] = (__bf16)p;
            }
        }
        ps += xor_lanes(ps, 16);
        ps += xor_lanes(ps, 32);
        lsum = lsum * alpha + ps;
        m = mn;

        // O^T[dim][head c] for this wave's dimensions; K index 8g + e of
        // product kk is key 32kk + 4g + e (e < 4) or 32kk + 16 + 4g + e - 4.
        const int trow = 4 * g + (c >> 2);
        const int tcol = dim0 + 4 * (c & 3);
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
            f32x4 acc = o[dt] * alpha;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const __bf16* base = vtile + (32 * kk + trow) * kVStride + tcol + 16 * dt;
                const bf16x4 lo = read_tr(base);
                const bf16x4 hi = read_tr(base + 16 * kVStride);
                const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[kk], acc, 0, 0, 0);
            }
            o[dt] = acc;
        }
    }

    if (!head_ok) return;
    if constexpr (DIRECT) {
        float f = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        if constexpr (KVF8) f *= *a.kv_scale;
        uint16_t* orow = a.out + ((size_t)b * a.H + head) * kValue + dim0;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
            const f32x4 v = o[dt] * f;
            const bf16x2 lo = {(__bf16)v.x, (__bf16)v.y}, hi = {(__bf16)v.z, (__bf16)v.w};
            *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * g) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
    } else {
        const size_t p = ((size_t)b * a.H + head) * a.splits + split;
        float* po = a.part_o + p * kValue + dim0;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt)
            *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
        if (w == 0 && g == 0) {
            a.part_m[p] = m;
            a.part_l[p] = lsum;
        }
    }
}

// Merge the key ranges of one (sequence, head): one wavefront, 8 value
// dimensions per lane.  Ranges without keys (sum 0) carry no weight.
template <bool KVF8>
__global__ void __launch_bounds__(64) mla_attn_combine_kernel(const Args a) {
    const int bh = blockIdx.x;              // b * H + h
    const int lane = threadIdx.x;
    const size_t p0 = (size_t)bh * a.splits;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
        if (a.part_l[p0 + s] > 0.0f) mx = fmaxf(mx, a.part_m[p0 + s]);
    float den = 0.0f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
        const float l = a.part_l[p0 + s];
        if (!(l > 0.0f)) continue;
        const float w = __builtin_amdgcn_exp2f(a.part_m[p0 + s] - mx);
        den += l * w;
        const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o + (p0 + s) * kValue + 8 * lane);
        const f32x4 v0 = po[0], v1 = po[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[e] += w * v0[e];
            acc[4 + e] += w * v1[e];
        }
    }
    float f = den > 0.0f ? 1.0f / den : 0.0f;
    if constexpr (KVF8) f *= *a.kv_scale;
    uint16_t r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = bf16_bits(acc[e] * f);
    u32x4 packed;
#pragma unroll
    for (int w = 0; w < 4; ++w) packed[w] = uint32_t(r[2 * w]) | (uint32_t(r[2 * w + 1]) << 16);
    *reinterpret_cast<u32x4*>(a.out + (size_t)bh * kValue + 8 * lane) = packed;
}

// ---- host side ---------------------------------------------------------------

int check_dims(const mla_attn_dims* d, uint32_t flags) {
    if (d == nullptr) return MLA_DQ_ERR_NULL;
    if (flags & ~(MLA_ATTN_Q_FP8 | MLA_ATTN_KV_FP8)) return MLA_DQ_ERR_FLAGS;
    if (d->batch < 0 || d->num_heads < 1 || d->num_blocks < 1 || d->block_size < 1 ||
        d->max_blocks_per_seq < 1 || d->max_seq_len < 0)
        return MLA_DQ_ERR_DIM;
    if (d->batch > INT32_MAX || d->num_heads > (1 << 20) || d->num_blocks > INT32_MAX ||
        d->block_size > (1 << 20) || d->max_blocks_per_seq > INT32_MAX)
        return MLA_DQ_ERR_DIM;
    if (d->max_seq_len > d->max_blocks_per_seq * d->block_size || d->max_seq_len > INT32_MAX / 2)
        return MLA_DQ_ERR_DIM;
    if (d->num_blocks > (INT64_MAX / 2048) / d->block_size) return MLA_DQ_ERR_DIM;
    return MLA_DQ_OK;
}

// Workgroups the key split aims for (two resident per CU); the environment
// variable MLA_ATTN_TARGET_WGS overrides it (read once per process).
int64_t target_workgroups() {
    static const int64_t v = [] {
        const char* e = getenv("MLA_ATTN_TARGET_WGS");
        if (e && *e) {
            char* end = nullptr;
            const long long x = strtoll(e, &end, 10);
            if (end && *end == '\0' && x >= 1 && x <= (1ll << 30)) return int64_t(x);
        }
        return int64_t(kTargetWorkgroupsDefault);
    }();
    return v;
}

int make_plan(const mla_attn_dims* d, uint32_t flags, mla_attn_plan* p) {
    const int rc = check_dims(d, flags);
    if (rc != MLA_DQ_OK) return rc;
    const int64_t head_tiles = (d->num_heads + 15) / 16;
    const int64_t steps = d->max_seq_len > 0 ? (d->max_seq_len + kStepKeys - 1) / kStepKeys : 1;
    const int64_t base = d->batch * head_tiles;
    const int64_t target = target_workgroups();
    int64_t splits = base > 0 ? (target + base - 1) / base : 1;
    if (splits < 1) splits = 1;
    if (splits > steps) splits = steps;
    const int64_t kps = ((steps + splits - 1) / splits) * kStepKeys;
    splits = d->max_seq_len > 0 ? (d->max_seq_len + kps - 1) / kps : 1;
    if (base * splits > INT32_MAX) return MLA_DQ_ERR_DIM;
    p->splits = int32_t(splits);
    p->keys_per_split = int32_t(kps);
    p->head_tiles = int32_t(head_tiles);
    p->combine = splits > 1 ? 1 : 0;
    p->workgroups = base * splits;
    p->workspace_bytes = p->combine ? d->batch * d->num_heads * splits * (kValue + 2) * 4 : 0;
    p->target_workgroups = target;
    p->xcd_remap = (head_tiles > 1 && p->workgroups % 8 == 0) ? 1 : 0;
    p->block_threads = kThreads;
    return MLA_DQ_OK;
}

bool aligned(const void* x, uintptr_t n) { return (reinterpret_cast<uintptr_t>(x) % n) == 0; }

template <bool QF8, bool KVF8>
hipError_t launch_pair(const Args& a, const mla_attn_plan& p, hipStream_t stream) {
    const dim3 grid(uint32_t(p.workgroups)), block(kThreads);
    if (!p.combine) {
        hipLaunchKernelGGL((mla_attn_partial_kernel<QF8, KVF8, true>), grid, block, 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((mla_attn_partial_kernel<QF8, KVF8, false>), grid, block, 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mla_attn_combine_kernel<KVF8>), dim3(uint32_t(a.B * a.H)), dim3(64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace mla_attn

extern "C" {

size_t mla_decode_attention_workspace_size(const mla_attn_dims* dims, uint32_t flags) {
    mla_attn_plan p;
    if (mla_attn::make_plan(dims, flags, &p) != MLA_DQ_OK) return 0;
    return size_t(p.workspace_bytes);
}

int mla_decode_attention_plan(const mla_attn_dims* dims, uint32_t flags, mla_attn_plan* plan) {
    if (plan == nullptr) return MLA_DQ_ERR_NULL;
    return mla_attn::make_plan(dims, flags, plan);
}

int mla_decode_attention(void* out, const void* q, const void* cache, const int32_t* block_table,
                         const int32_t* seq_lens, const float* q_scale, const float* kv_scale,
                         float sm_scale, void* workspace, size_t workspace_bytes, uint32_t flags,
                         const mla_attn_dims* dims, void* stream) {
    using namespace mla_attn;
    mla_attn_plan p;
    int rc = make_plan(dims, flags, &p);
    if (rc != MLA_DQ_OK) return rc;
    if (dims->batch == 0) return MLA_DQ_OK;
    const bool qf8 = flags & MLA_ATTN_Q_FP8, kvf8 = flags & MLA_ATTN_KV_FP8;
    if (!out || !q || !cache || !block_table || !seq_lens) return MLA_DQ_ERR_NULL;
    if ((qf8 && !q_scale) || (kvf8 && !kv_scale)) return MLA_DQ_ERR_NULL;
    if (p.workspace_bytes > 0 && !workspace) return MLA_DQ_ERR_NULL;
    if (workspace_bytes < size_t(p.workspace_bytes)) return MLA_ATTN_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || (workspace && !aligned(workspace, 16)) ||
        (qf8 && !aligned(q_scale, 4)) || (kvf8 && !aligned(kv_scale, 4)))
        return MLA_DQ_ERR_ALIGN;
    if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return MLA_DQ_ERR_DIM;

    Args a;
    a.out = static_cast<uint16_t*>(out);
    a.q = static_cast<const uint8_t*>(q);
    a.cache = static_cast<const uint8_t*>(cache);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.q_scale = q_scale;
    a.kv_scale = kv_scale;
    const int64_t parts = dims->batch * dims->num_heads * int64_t(p.splits);
    a.part_o = static_cast<float*>(workspace);
    a.part_m = a.part_o ? a.part_o + parts * kValue : nullptr;
    a.part_l = a.part_m ? a.part_m + parts : nullptr;
    a.score_scale = sm_scale * 1.4426950408889634f;
    a.B = int32_t(dims->batch);
    a.H = int32_t(dims->num_heads);
    a.num_blocks = int32_t(dims->num_blocks);
    a.block_size = int32_t(dims->block_size);
    a.max_blocks = int32_t(dims->max_blocks_per_seq);
    a.max_seq_len = int32_t(dims->max_seq_len);
    a.splits = p.splits;
    a.keys_per_split = p.keys_per_split;
    a.head_tiles = p.head_tiles;
    a.xcd_remap = p.xcd_remap;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (qf8)
        e = kvf8 ? launch_pair<true, true>(a, p, s) : launch_pair<true, false>(a, p, s);
    else
        e = kvf8 ? launch_pair<false, true>(a, p, s) : launch_pair<false, false>(a, p, s);
    return e == hipSuccess ? MLA_DQ_OK : MLA_DQ_ERR_LAUNCH;
}

}  // extern "C"
