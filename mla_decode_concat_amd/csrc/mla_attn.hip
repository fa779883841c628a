// MLA decode attention over the paged latent cache for gfx950 (MI355X).
//
// The definition is in include/mla_attn.h.  Split-KV decoding: a workgroup
// handles one (sequence, tile of 16 heads, range of keys) with four compute
// wavefronts.  They work independently on interleaved tiles of 16 keys (wave
// w takes tiles w, w+4, w+8, ... of the range), each with its own online
// softmax and its own accumulator for all 512 value dimensions, and meet
// once at the end to merge their four partial results through LDS.
//
// Three kernels share that scheme.  With a bf16 cache each compute
// wavefront loads its own keys into registers (mla_attn_partial_kernel,
// described next).  With an E4M3 cache four loader wavefronts stream the
// keys into an LDS ring for their compute partners (mla_attn_ring_kernel,
// further down), except for ranges of one tile per compute wavefront, whose
// wavefronts copy their tile into LDS themselves (mla_attn_short_kernel).
//
// Per pair of 16-key tiles, in one wavefront (lane l: c = l % 16, g = l / 16):
//  * scores on the matrix cores, transposed: S^T[key][head] = K Q^T with
//    v_mfma_f32_16x16x32_bf16 over 18 steps of 32 of the 576 dimensions.
//    Lane l loads 16 bytes of key c per instruction: bf16 dimensions
//    32s + 8g .. +7 for step s (the E4M3 kernel: dimensions 64i + 16g .. +15,
//    which feed steps 2i (first eight) and 2i + 1 (last eight); the sum over
//    the 576 dimensions does not care how they are dealt to steps and K
//    slots).  Operand B is head c's query at the same dimensions, read from
//    the workgroup's query tile in LDS.  The result leaves lane l with head
//    c's scores for keys 4g .. 4g+3 of the tile.
//  * each tile's value part (first 512 elements) goes, as bf16, to a
//    wavefront-private LDS tile in the cache's row-major layout, and the
//    tile's registers reload with the next pair's keys.
//  * online softmax in base 2.  The running max only moves when a pair's
//    max exceeds it by more than 8 (the weights then stay below 2^8; exact
//    ratios are unaffected), so the 128 accumulators are rarely rescaled.
//  * values on the matrix cores: O^T[dim][head] += V^T P^T with
//    v_mfma_f32_16x16x32_bf16 over 32 tiles of 16 dimensions, 32 keys per
//    product.  K index 8g + e is key 4g + e of the first tile (e < 4) or
//    key 4g + e - 4 of the second, so operand B (P^T) is the lane's own
//    eight weights, and operand A (V^T) is two ds_read_b64_tr_b16 of the
//    row-major tiles: in each 16-lane group that load hands lane j column j
//    of the four rows the group's lanes address (lane i: row i / 4,
//    columns 4(i % 4) .. +3).
//
// E4M3 operands (queries in both kernels, keys and values in the ring
// kernel) convert exactly to bf16 (3 mantissa bits, two values per
// v_cvt_scalef32_pk_bf16_fp8 with scale 1); their scales are applied in
// fp32 to the scores and to the result.  With one range per
// sequence the workgroup writes the bf16 output itself; otherwise it writes
// (max, sum, unnormalised output) to the workspace and a second kernel merges
// the ranges.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "mla_attn.h"
#include "mla_dq.h"

namespace mla_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRow = 576;           // latent row: 512 value + 64 positional elements
constexpr int kValue = 512;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;                // keys per wavefront tile
constexpr int kStepKeys = kTile * kWaves;  // keys the workgroup covers per round
constexpr int kSteps = kRow / 32;        // 18 score products of 32 dimensions
constexpr int kVSteps = kValue / 32;     // 16 of them cover the value part
constexpr int kDimTiles = kValue / 16;   // 32 value products of 16 dimensions
// bf16 elements per LDS row of a value tile: 512 + 16 of padding puts the
// four rows a 16-lane group reads in one transpose load on disjoint banks.
constexpr int kVStride = kValue + 16;
constexpr int kWaveTile = 2 * kTile * kVStride;       // bf16 elements per wavefront (two tiles)
// bf16 elements per LDS row of the query tile: 576 + 8 of padding keeps the
// 16 rows one instruction reads on disjoint banks.
constexpr int kQStride = kRow + 8;
constexpr int kLdsBytes = kWaves * kWaveTile * 2;     // 135168: covers the merge buffer too
static_assert(kWaves * 24 * 64 * 16 <= kLdsBytes, "merge buffer");
constexpr int kTargetWorkgroupsDefault = 256;  // one resident workgroup per CU
constexpr int kMaxSplits = 1024;               // key ranges per sequence, at most
constexpr int kMinSplitSteps = 1;              // 64-key rounds per range, at least
// Partial outputs of at least this many bytes per call are stored
// non-temporally (measured, µs per call with cold caches: E4M3 64 x 4096 keys
// 39.3 -> 36.9-37.5, 32 x 2048 keys 19.1-19.4 -> 17.8-18.1; bf16 64 x 4096
// 64.7 -> 64.1).  With fewer the merge kernel's reads of them slow down more
// than the stores gain (1 x 1024 keys 10.5 -> 11.0).  A kernel instance per
// choice: with a run-time branch the compiler merges the two stores and drops
// the non-temporal hint.
constexpr int64_t kStreamPartialBytes = 4ll << 20;
// The running max moves only when a pair of tiles exceeds it by more than
// this (log2 units).
constexpr float kRebase = 8.0f;

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
    int32_t grid;        // workgroups of the range kernel (read with the other
                         // arguments, not from the dispatch's implicit ones)
};

// Eight E4M3 codes -> eight bf16, two per v_cvt_scalef32_pk_bf16_fp8 with
// scale 1 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 raw) {
    bf16x8 r;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, true);
        r[4 * w + 0] = lo[0];
        r[4 * w + 1] = lo[1];
        r[4 * w + 2] = hi[0];
        r[4 * w + 3] = hi[1];
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

// A key tile in registers: 16 bytes per load instruction and lane, 18
// instructions for a bf16 row, 9 for an E4M3 row.
template <bool FP8>
struct KeyTile {
    static constexpr int kLoads = FP8 ? kSteps / 2 : kSteps;
    u32x4 r[kLoads];
    // first element of load i for lane group g
    static __device__ __forceinline__ int dim(int i, int g) { return FP8 ? 64 * i + 16 * g : 32 * i + 8 * g; }
    // operand A of score step s, as bf16
    __device__ __forceinline__ bf16x8 step(int s) const {
        if constexpr (FP8)
            return e4m3x8_to_bf16(s & 1 ? u32x2{r[s >> 1][2], r[s >> 1][3]} : u32x2{r[s >> 1][0], r[s >> 1][1]});
        else
            return __builtin_bit_cast(bf16x8, r[s]);
    }
    // Score step s takes the 8-element chunk 8(s / 2) + 2g + s % 2 (E4M3) or
    // 4s + g (bf16) of the row: the lane part plus a constant offset.
    static __device__ __forceinline__ int lane_dim(int g) { return FP8 ? 16 * g : 8 * g; }
    static constexpr int step_dim(int s) { return FP8 ? 64 * (s >> 1) + 8 * (s & 1) : 32 * s; }
};

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per 16-lane
// row): v_permlane16_swap and v_permlane32_swap hand each lane its partner
// row's value without going through LDS.
__device__ __forceinline__ float max_rows(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float m = fmaxf(__builtin_bit_cast(float, (unsigned)a[0]),
                          __builtin_bit_cast(float, (unsigned)a[1]));
    const unsigned w = __builtin_bit_cast(unsigned, m);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}

__device__ __forceinline__ float sum_rows(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float m = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
    const unsigned w = __builtin_bit_cast(unsigned, m);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
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
        const int n = a.grid;                // a multiple of 8 when remapping
        x = (x % 8) * (n / 8) + x / 8;
    }
    ht = x % a.head_tiles;
    const int rest = x / a.head_tiles;
    split = rest % a.splits;
    b = rest / a.splits;
}

template <bool FP8>
__device__ __forceinline__ void load_tile(KeyTile<FP8>& kt, const uint8_t* row, int g) {
#pragma unroll
    for (int i = 0; i < KeyTile<FP8>::kLoads; ++i)
        kt.r[i] = *reinterpret_cast<const u32x4*>(row + KeyTile<FP8>::dim(i, g) * (FP8 ? 1 : 2));
}

template <bool FP8>
struct PairRegs {
    KeyTile<FP8> t[2];
};

// The workgroup's 16 query rows (heads 16 ht .. 16 ht + 15 of sequence b) as
// bf16 in LDS, row stride kQStride; rows for heads past H are zero.  The NT
// staging threads first issue all their loads (unconditionally, at clamped
// rows) and only then write, so the loads share one memory latency; a
// kernel may issue other loads between the two halves.
template <bool QF8, int NT>
struct QueryStage {
    static constexpr int kChunks = 16 * (kRow / 8);   // 8-element chunks of the tile
    static constexpr int kIter = (kChunks + NT - 1) / NT;
    Chunk<QF8> v[kIter];

    __device__ __forceinline__ void load(const Args& a, int b, int ht, int tid) {
        const size_t q_row_bytes = (size_t)kRow * (QF8 ? 1 : 2);
#pragma unroll
        for (int k = 0; k < kIter; ++k) {
            int idx = tid + NT * k;
            idx = idx < kChunks ? idx : kChunks - 1;
            const int hq = idx / (kRow / 8), ch = idx % (kRow / 8);
            int hh = ht * 16 + hq;
            hh = hh < a.H ? hh : a.H - 1;
            v[k] = load_chunk<QF8>(a.q + ((size_t)b * a.H + hh) * q_row_bytes, 8 * ch);
        }
    }
    __device__ __forceinline__ void store(const Args& a, int ht, __bf16* qlds, int tid) const {
#pragma unroll
        for (int k = 0; k < kIter; ++k) {
            const int idx = tid + NT * k;
            if (idx < kChunks) {
                const int hq = idx / (kRow / 8), ch = idx % (kRow / 8);
                const bf16x8 x = ht * 16 + hq < a.H ? to_bf16<QF8>(v[k]) : bf16x8{};
                *reinterpret_cast<bf16x8*>(qlds + hq * kQStride + 8 * ch) = x;
            }
        }
    }
};

template <bool QF8, int NT>
__device__ __forceinline__ void stage_queries(const Args& a, int b, int ht, __bf16* qlds, int tid) {
    QueryStage<QF8, NT> qs;
    qs.load(a, b, ht, tid);
    __builtin_amdgcn_sched_barrier(0);
    qs.store(a, ht, qlds, tid);
}

// Workgroup barrier for LDS traffic only: this wavefront's LDS operations are
// complete, global loads and stores may still be in flight (__syncthreads
// would also wait for those).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Merge the four compute wavefronts' (max, sum, output) through LDS with
// weights 2^(m_w - M) over the workgroup max M, then write the range's result:
// bf16 output when the range is the whole sequence, else the unnormalised
// output with its max and sum.  Threads 0..255 are the compute wavefronts;
// the others only pass the barriers.  One pass: compute wavefront w owns
// value-dim tiles 8w .. 8w+7 (dims 128w .. 128w+127).  It stores the other
// 24 of its 32 accumulator tiles to LDS, lane-major (tile slot k of wave v,
// lane l at 16 B * (64 (24 v + k) + l), so every store and load instruction
// covers 1 KB of consecutive LDS), and sums its own tiles from registers with
// the three others' from LDS.  mb is LDS scratch of at least 96 KB that no
// wavefront reads any more.
template <bool KVF8, bool DIRECT, bool STREAMP, int NT>
__device__ __forceinline__ void merge_waves(const Args& a, const f32x4 (&o)[kDimTiles], float m, float lsum,
                                            bool compute, int b, int split, int ht, float* mb,
                                            float (&mls)[2][kWaves][16]) {
    constexpr int kOwn = kDimTiles / kWaves;                  // 8 tiles per wavefront
    constexpr int kShared = kDimTiles - kOwn;                 // 24 tiles stored to LDS
    const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
    const int w = (threadIdx.x >> 6) & (kWaves - 1);
    if (compute && g == 0) {
        mls[0][w][c] = m;
        mls[1][w][c] = lsum;
    }
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
        if (mls[1][v][c] > 0.0f) M = fmaxf(M, mls[0][v][c]);
    const float own = lsum > 0.0f ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
    float Ltot = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const float lv = mls[1][v][c];
        if (lv > 0.0f) Ltot += lv * __builtin_amdgcn_exp2f(mls[0][v][c] - M);
    }
    f32x4* lm = reinterpret_cast<f32x4*>(mb);
    if (compute) {
#pragma unroll
        for (int j = 0; j < kDimTiles; ++j) {
            if (j / kOwn != w) {
                const int k = j < kOwn * w ? j : j - kOwn;
                lm[64 * (kShared * w + k) + lane] = o[j] * own;
            }
        }
    }
    lds_barrier();
    if (!compute) return;
    const bool head_ok = ht * 16 + c < a.H;
    float fin = 1.0f;
    if constexpr (DIRECT) {
        fin = Ltot > 0.0f ? 1.0f / Ltot : 0.0f;
        if constexpr (KVF8) fin *= *a.kv_scale;
    }
    const size_t row = (size_t)b * a.H + ht * 16 + c;       // (sequence, head) of this lane
    const size_t p = row * a.splits + split;
#pragma unroll
    for (int j = 0; j < kDimTiles; ++j) {
        if (j / kOwn != w) continue;
        f32x4 acc = o[j] * own;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v == w) continue;
            const int k = j < kOwn * v ? j : j - kOwn;
            acc += lm[64 * (kShared * v + k) + lane];
        }
        if (head_ok) {
            const int d0 = 16 * j + 4 * g;
            if constexpr (DIRECT) {
                const f32x4 r = acc * fin;
                const bf16x2 lo = {(__bf16)r.x, (__bf16)r.y}, hi = {(__bf16)r.z, (__bf16)r.w};
                *reinterpret_cast<u32x2*>(a.out + row * kValue + d0) =
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            } else {
                f32x4* dst = reinterpret_cast<f32x4*>(a.part_o + p * kValue + d0);
                if constexpr (STREAMP)
                    __builtin_nontemporal_store(acc, dst);
                else
                    *dst = acc;
            }
        }
    }
    if constexpr (!DIRECT) {
        if (threadIdx.x < 16 && head_ok) {
            a.part_m[p] = M;
            a.part_l[p] = Ltot;
        }
    }
}

template <bool QF8, bool DIRECT, bool STREAMP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_attn_partial_kernel(const Args a) {
    constexpr bool KVF8 = false;   // bf16 cache (E4M3 caches go to mla_attn_ring_kernel)
    // Pairs of key tiles held in registers per wavefront.  Each tile of the
    // pair reloads (with the pair kPB ahead) as soon as its scores and value
    // rows are out of its registers.  More pairs in flight make the compiler
    // park key rows in accumulator registers and copy them back (measured
    // slower).
    constexpr int kPB = 1;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
    __shared__ __attribute__((aligned(16))) __bf16 qlds[16 * kQStride];
    __shared__ float mls[2][kWaves][16];

    int b, split, ht;
    decode_wg(a, b, split, ht);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int k0 = split * a.keys_per_split;
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int k1 = (k0 + a.keys_per_split < L) ? k0 + a.keys_per_split : L;
    // Tiles of this wavefront: keys k0 + 16 (w + 4t) .. +15; pair p is tiles
    // 2p and 2p + 1.
    const int first = k0 + kTile * w;
    const int nt = k1 > first ? (k1 - first + kStepKeys - 1) / kStepKeys : 0;
    const int np = (nt + 1) / 2;

    // The query loads go out first, then the first pair's block-table entries
    // and keys.  Block-table entries are read at keys clamped to
    // max_seq_len - 1 only, so they wait for nothing but the table (not for
    // the sequence length).  Every tile of a pair goes through the value
    // product, so every row read must be finite: a lane whose key lies past
    // the range reads the tile's first key (lane 0's page), and a tile wholly
    // past the range reads the range's first key.  Pairs from 1 on that lie
    // past the range (requested only to keep the loads unconditional) repeat
    // the range's last tile.
    QueryStage<QF8, kThreads> qs;
    qs.load(a, b, ht, threadIdx.x);
    const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
    const size_t row_bytes = (size_t)kRow * (KVF8 ? 1 : 2);
    const int last = k1 > 0 ? k1 - 1 : 0;
    const int kmax = a.max_seq_len > 0 ? a.max_seq_len - 1 : 0;
    auto tile_at = [&](int t) -> int { return t < 2 || t < nt ? t : (nt > 0 ? nt - 1 : 0); };
    auto spec_key = [&](int t) -> int {
        const int key = first + kStepKeys * tile_at(t) + c;
        return key < kmax ? key : kmax;
    };
    auto page_of = [&](int t) -> int { return bt[spec_key(t) / a.block_size]; };
    int page_first = 0;   // page of the range's first key (lane 0 of tile 0)
    auto row_of = [&](int t, int page) -> const uint8_t* {
        const int raw = first + kStepKeys * tile_at(t) + c, raw0 = raw - c;
        int key = raw < kmax ? raw : kmax;
        if (raw > last) {
            if (raw0 <= last) {
                key = raw0;
                page = __builtin_amdgcn_readlane(page, 0);
            } else {
                key = first < kmax ? first : kmax;
                page = page_first;
            }
        }
        page = page < 0 ? 0 : (page >= a.num_blocks ? a.num_blocks - 1 : page);
        return a.cache + ((size_t)page * a.block_size + key % a.block_size) * row_bytes;
    };

    PairRegs<KVF8> kc[kPB];
    int pg[kPB][2];
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
        pg[j][0] = page_of(2 * j);
        pg[j][1] = page_of(2 * j + 1);
    }
    page_first = __builtin_amdgcn_readlane(pg[0][0], 0);
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            load_tile<KVF8>(kc[j].t[h], row_of(2 * j + h, pg[j][h]), g);
            pg[j][h] = page_of(2 * (j + kPB) + h);
        }
    }

    // The tile's 16 query rows, as bf16, in LDS: operand B of the score
    // products is read from there.
    qs.store(a, ht, qlds, threadIdx.x);
    __syncthreads();
    const __bf16* qrow = qlds + c * kQStride + KeyTile<KVF8>::lane_dim(g);
    float sc = a.score_scale;
    if constexpr (QF8) sc *= *a.q_scale;
    if constexpr (KVF8) sc *= *a.kv_scale;

    f32x4 o[kDimTiles];
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.0f;
    __bf16* vt = reinterpret_cast<__bf16*>(smem) + w * kWaveTile;
    // Rows 0..15: the pair's first tile, rows 16..31: its second.
    // The tile's 16-byte chunk j of row r sits at chunk j ^ ((r >> 3) & 1): the
    // 16 rows one store instruction writes then cover all 64 banks, and the
    // four rows of a transpose load keep theirs (the swap stays inside each
    // row's 32-byte column block).
    // Where score step s's 8 value elements go in row c: chunk index j (the
    // lane part plus step_dim(s) / 8) becomes j ^ (c >> 3).
    int vsw[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
        vsw[par] = 8 * ((KeyTile<KVF8>::lane_dim(g) / 8 + (KVF8 ? par : 0)) ^ (c >> 3));
    const __bf16* trow = vt + (4 * g + (c >> 2)) * kVStride +
                         8 * (((c & 3) >> 1) ^ ((g >> 1) & 1)) + 4 * (c & 1);

    auto process = [&](int j, int p) {
        f32x4 sc2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __bf16* vrow = vt + (16 * h + c) * kVStride;
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const bf16x8 kb = kc[j].t[h].step(s);
                const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qrow + KeyTile<KVF8>::step_dim(s));
                if (s & 1)
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, s1, 0, 0, 0);
                else
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, s0, 0, 0, 0);
                if (s < kVSteps)
                    *reinterpret_cast<bf16x8*>(vrow + (KeyTile<KVF8>::step_dim(s) & ~15) + vsw[s & 1]) = kb;
            }
            sc2[h] = s0 + s1;
            // This tile's registers are free: the pair kPB ahead streams in.
            if (p + kPB < np)
                load_tile<KVF8>(kc[j].t[h], row_of(2 * (p + kPB) + h, pg[j][h]), g);
            pg[j][h] = page_of(2 * (p + 2 * kPB) + h);
        }
        float sv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key0 = first + kStepKeys * (2 * p + h) + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sv[4 * h + i] = key0 + i < k1 ? sc2[h][i] * sc : -INFINITY;
        }
        float tm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        tm = max_rows(tm);
        if (__builtin_amdgcn_ballot_w64(tm > m + kRebase) != 0) {
            const float mn = tm > m + kRebase ? tm : m;
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt) o[dt] *= alpha;
            lsum *= alpha;
            m = mn;
        }
        // Operand B of the value product: K index 8g + e is key 4g + e of the
        // pair's first tile (e < 4) or key 4g + e - 4 of its second.
        float ps = 0.0f;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(sv[e] - m);
            ps += pe;
            pb[e] = (__bf16)pe;
        }
        lsum += sum_rows(ps);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
            const bf16x4 lo = read_tr(trow + 16 * dt);
            const bf16x4 hi = read_tr(trow + 16 * kVStride + 16 * dt);
            const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[dt], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    };

    for (int p0 = 0; p0 < np; p0 += kPB) {
#pragma unroll
        for (int j = 0; j < kPB; ++j)
            if (p0 + j < np) process(j, p0 + j);
    }

    merge_waves<KVF8, DIRECT, STREAMP, kThreads>(a, o, m, lsum, true, b, split, ht, reinterpret_cast<float*>(smem),
                                                 mls);
}

// ---- E4M3 cache: loader and compute wavefronts over an LDS ring -------------
//
// With an E4M3 cache a compute wavefront spends most of its time blocked on
// issuing its own key loads when it is the only wavefront on its SIMD.  Here
// each SIMD runs one compute wavefront and one loader wavefront.  The loader
// streams the raw E4M3 key tiles of its compute partner (the same tiles
// w, w + 4, ... of the range) through registers into a three-slot LDS ring
// and never computes; the compute wavefront only reads LDS.
//
// Ring slot layout: one 16-key tile as 9 blocks of 1 KB; block i holds, at
// 16 l, the 16 bytes of key c = l % 16 at row bytes 64 i + 16 (l / 16): the
// loader's lane l writes what its own 16-byte load i returned, and the score
// step reads it back with the same lane mapping (both 1 KB contiguous).
// Byte d of key k therefore sits at 256 (d / 16) + 16 k + d % 16.
//
// The value product takes one 16-key tile with v_mfma_f32_16x16x16_bf16:
// lane (c, g) needs dims 16 dt + c of keys 4g .. 4g+3.  One ds_read_b64_tr_b8
// serves two dim tiles: in each 16-lane group it hands lane j byte j % 8 of
// the 8-byte chunks of lanes 2e + j / 8 (e = 0..7).  Lane i = c of group g
// therefore addresses key 4g + (i / 2) % 4 at dims 16 (2dd + i / 8) + 8 (i % 2):
// lane j receives keys 4g .. 4g+3 at dim 32 dd + j in bytes 0..3 and at dim
// 32 dd + 16 + j in bytes 4..7.
//
// Handshake (LDS counters, one pair per compute wavefront): ready = tiles
// written, done = tiles consumed.  A tile goes to slot t % 3 once done
// reaches t - 2.  LDS executes each wavefront's operations in order, so a
// counter written after the data (or after the reads of a slot) is seen no
// earlier than them; the explicit lgkmcnt(0) waits make that hold across
// wavefronts too.
constexpr int kRingSlots = 3;
constexpr int kTileBytes = kTile * kRow;                       // 9216 bytes of E4M3
constexpr int kRingBytes = kWaves * kRingSlots * kTileBytes;   // 110592
constexpr int kRingThreads = 2 * kThreads;
static_assert(kWaves * 24 * 64 * 16 <= kRingBytes, "merge buffer inside the ring");

__device__ __forceinline__ int lds_counter(const int* p) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

__device__ __forceinline__ void lds_publish(int* p, int v) {
    // this wavefront's earlier LDS operations are done (and stay before the store)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Four E4M3 codes -> four bf16 (exact).
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16(uint32_t word) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
    return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

// One 16-key E4M3 tile in LDS (the ring slot layout: block i of 1 KB holds
// at 16 l the 16 bytes of key l % 16 at row bytes 64 i + 16 (l / 16))
// through one compute wavefront's scores, online softmax and value product.
// The tile holds keys first + 64 t .. +15; keys from k1 on weigh zero.
__device__ __forceinline__ void e4m3_tile(const uint8_t* base, const __bf16* qrow, int lane, int g, int vlane,
                                          float sc, int first, int t, int k1, f32x4 (&o)[kDimTiles], float& m,
                                          float& lsum) {
    // All of the tile's LDS reads go out first (keys for the scores,
    // transposed values for the value product), so their latency
    // overlaps instead of stalling each product in turn.
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    u32x4 kraw[kSteps / 2];
    i32x2 vraw[kDimTiles / 2];
#pragma unroll
    for (int i = 0; i < kSteps / 2; ++i)
        kraw[i] = *reinterpret_cast<const u32x4*>(base + 1024 * i + 16 * lane);
#pragma unroll
    for (int dd = 0; dd < kDimTiles / 2; ++dd)
        vraw[dd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + vlane + 512 * dd));
    __builtin_amdgcn_sched_barrier(0);
    // scores: S^T = K Q^T over 18 steps of 32 dims
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kSteps / 2; ++i) {
        const u32x4 raw = kraw[i];
        const bf16x8 ka = e4m3x8_to_bf16(u32x2{raw[0], raw[1]});
        const bf16x8 kb = e4m3x8_to_bf16(u32x2{raw[2], raw[3]});
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qrow + 64 * i);
        const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qrow + 64 * i + 8);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qa, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, s1, 0, 0, 0);
    }
    const f32x4 st = s0 + s1;
    const int key0 = first + kStepKeys * t + 4 * g;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = key0 + i < k1 ? st[i] * sc : -INFINITY;
    float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    tm = max_rows(tm);
    if (__builtin_amdgcn_ballot_w64(tm > m + kRebase) != 0) {
        const float mn = tm > m + kRebase ? tm : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) o[dt] *= alpha;
        lsum *= alpha;
        m = mn;
    }
    float ps = 0.0f;
    bf16x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(sv[e] - m);
        ps += pe;
        pb[e] = (__bf16)pe;
    }
    lsum += sum_rows(ps);
    // values: O^T += V^T P^T, two dim tiles per transpose load
#pragma unroll
    for (int dd = 0; dd < kDimTiles / 2; ++dd) {
        const i32x2 v = vraw[dd];
        o[2 * dd] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(e4m3x4_to_bf16(uint32_t(v[0])), pb,
                                                              o[2 * dd], 0, 0, 0);
        o[2 * dd + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(e4m3x4_to_bf16(uint32_t(v[1])), pb,
                                                                  o[2 * dd + 1], 0, 0, 0);
    }
}

template <bool QF8, bool DIRECT, bool STREAMP>
__global__ void __launch_bounds__(kRingThreads) mla_attn_ring_kernel(const Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
    __shared__ __attribute__((aligned(16))) __bf16 qlds[16 * kQStride];
    __shared__ float mls[2][kWaves][16];
    __shared__ int ready[kWaves], done[kWaves];

    int b, split, ht;
    decode_wg(a, b, split, ht);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = wave & (kWaves - 1);          // compute wavefront served or run
    const bool loader = wave >= kWaves;
    const int c = lane & 15, g = lane >> 4;
    const int k0 = split * a.keys_per_split;
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int k1 = (k0 + a.keys_per_split < L) ? k0 + a.keys_per_split : L;
    const int first = k0 + kTile * w;
    const int nt = k1 > first ? (k1 - first + kStepKeys - 1) / kStepKeys : 0;
    uint8_t* const slots = ring + w * kRingSlots * kTileBytes;

    if (threadIdx.x < kWaves) {
        ready[threadIdx.x] = 0;
        done[threadIdx.x] = 0;
    }

    // Loader state.  Its first pages and keys are requested before the
    // workgroup barrier, while the compute wavefronts stage the queries, and
    // before the sequence length is known: keys are clamped to
    // max_seq_len - 1 only, so every block-table entry and row read stays in
    // bounds.  Rows of keys past the range may hold anything (NaN included);
    // the loader writes zeros for them into the ring (only the range's last
    // tile has such keys), so a zero weight always meets finite data.  Tiles
    // from 2 on that lie past the range (requested only to keep the loads
    // unconditional, never handed over) repeat the range's last tile, which
    // is still in cache.
    const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
    const int last = k1 > 0 ? k1 - 1 : 0;
    const int kmax = a.max_seq_len > 0 ? a.max_seq_len - 1 : 0;
    auto tile_at = [&](int t) -> int { return t < 2 || t < nt ? t : (nt > 0 ? nt - 1 : 0); };
    auto key_of = [&](int t) -> int {
        const int key = first + kStepKeys * tile_at(t) + c;
        return key < kmax ? key : kmax;
    };
    auto page_of = [&](int t) -> int { return bt[key_of(t) / a.block_size]; };
    auto row_of = [&](int t, int page) -> const uint8_t* {
        page = page < 0 ? 0 : (page >= a.num_blocks ? a.num_blocks - 1 : page);
        return a.cache + ((size_t)page * a.block_size + key_of(t) % a.block_size) * kRow;
    };
    // Loads are unconditional: with no load on a branch the compiler's load
    // counters stay exact and it never waits for more than the data it needs.
    KeyTile<true> r0, r1;
    int pga = 0, pgb = 0;
    if (loader) {
        pga = page_of(0);
        pgb = page_of(1);
        load_tile<true>(r0, row_of(0, pga), g);
    } else {
        stage_queries<QF8, kThreads>(a, b, ht, qlds, threadIdx.x);
    }
    lds_barrier();

    f32x4 o[kDimTiles];
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.0f;

    if (loader) {
        auto put = [&](int u, const KeyTile<true>& cur) {
            while (lds_counter(&done[w]) < u - (kRingSlots - 1)) __builtin_amdgcn_s_sleep(1);
            asm volatile("" ::: "memory");
            uint8_t* dst = slots + (u % kRingSlots) * kTileBytes + 16 * lane;
            const bool past = first + kStepKeys * u + c > last;   // key past the range
#pragma unroll
            for (int i = 0; i < KeyTile<true>::kLoads; ++i)
                *reinterpret_cast<u32x4*>(dst + 1024 * i) = past ? u32x4{0u, 0u, 0u, 0u} : cur.r[i];
            lds_publish(&ready[w], u + 1);
        };
        for (int u = 0; u < nt; u += 2) {
            // tile u is in r0; tile u + 1 streams into r1, page u + 2 into pga
            pga = page_of(u + 2);
            load_tile<true>(r1, row_of(u + 1, pgb), g);
            put(u, r0);
            // tile u + 1 is in r1; tile u + 2 streams into r0, page u + 3 into pgb
            pgb = page_of(u + 3);
            load_tile<true>(r0, row_of(u + 2, pga), g);
            if (u + 1 < nt) put(u + 1, r1);
        }
    } else {
        float sc = a.score_scale * *a.kv_scale;
        if constexpr (QF8) sc *= *a.q_scale;
        const __bf16* qrow = qlds + c * kQStride + 16 * g;
        const int vlane = 256 * (c >> 3) + 64 * g + 8 * (c & 7);
        for (int t = 0; t < nt; ++t) {
            while (lds_counter(&ready[w]) <= t) __builtin_amdgcn_s_sleep(1);
            asm volatile("" ::: "memory");
            const uint8_t* base = slots + (t % kRingSlots) * kTileBytes;
            e4m3_tile(base, qrow, lane, g, vlane, sc, first, t, k1, o, m, lsum);
            lds_publish(&done[w], t + 1);
        }
    }

    merge_waves<true, DIRECT, STREAMP, kRingThreads>(a, o, m, lsum, !loader, b, split, ht,
                                                     reinterpret_cast<float*>(ring), mls);
}

// Ranges of one tile per compute wavefront (64 keys, the plan's shortest):
// no loader wavefronts.  Each of the four wavefronts copies its own tile from
// memory straight into LDS (global_load_lds_dwordx4: lane l's 16 bytes land
// at 16 l, which is the ring slot layout), so the tile takes no register hop
// and no handshake.  Block-table and row reads use keys clamped to
// max_seq_len - 1, as the ring kernel's loaders do, so they go out before the
// sequence length arrives; the wavefront then zeroes the rows of keys past
// the range, so that a zero weight meets finite data.  The 96 KB buffer holds
// the four tiles first and the merge's exchange afterwards.
template <bool QF8, bool DIRECT, bool STREAMP>
__global__ void __launch_bounds__(kThreads) mla_attn_short_kernel(const Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[kWaves * 24 * 64 * 16];
    __shared__ __attribute__((aligned(16))) __bf16 qlds[16 * kQStride];
    __shared__ float mls[2][kWaves][16];
    static_assert(kWaves * kTileBytes <= kWaves * 24 * 64 * 16, "tiles inside the merge buffer");

    int b, split, ht;
    decode_wg(a, b, split, ht);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int first = split * a.keys_per_split + kTile * w;
    const int kmax = a.max_seq_len > 0 ? a.max_seq_len - 1 : 0;
    const int key = first + c < kmax ? first + c : kmax;
    int page = a.block_table[(size_t)b * a.max_blocks + key / a.block_size];
    QueryStage<QF8, kThreads> qs;
    qs.load(a, b, ht, threadIdx.x);
    int L = a.seq_lens[b];
    page = page < 0 ? 0 : (page >= a.num_blocks ? a.num_blocks - 1 : page);
    const uint8_t* row = a.cache + ((size_t)page * a.block_size + key % a.block_size) * kRow;
    uint8_t* const slot = buf + w * kTileBytes;
#pragma unroll
    for (int i = 0; i < kSteps / 2; ++i)
        __builtin_amdgcn_global_load_lds(row + 64 * i + 16 * g, (lds_void*)(slot + 1024 * i), 16, 0, 0);
    qs.store(a, ht, qlds, threadIdx.x);
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int k0 = split * a.keys_per_split;
    const int k1 = (k0 + a.keys_per_split < L) ? k0 + a.keys_per_split : L;
    float sc = a.score_scale * *a.kv_scale;
    if constexpr (QF8) sc *= *a.q_scale;
    // the tile is in LDS once this wavefront's loads are done; rows of keys
    // past the range are overwritten only after that
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (first + c >= k1) {
#pragma unroll
        for (int i = 0; i < kSteps / 2; ++i)
            *reinterpret_cast<u32x4*>(slot + 1024 * i + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
    }
    lds_barrier();

    f32x4 o[kDimTiles];
#pragma unroll
    for (int dt = 0; dt < kDimTiles; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.0f;
    if (k1 > first) {
        const __bf16* qrow = qlds + c * kQStride + 16 * g;
        const int vlane = 256 * (c >> 3) + 64 * g + 8 * (c & 7);
        e4m3_tile(slot, qrow, lane, g, vlane, sc, first, 0, k1, o, m, lsum);
    }
    merge_waves<true, DIRECT, STREAMP, kThreads>(a, o, m, lsum, true, b, split, ht, reinterpret_cast<float*>(buf),
                                                  mls);
}

// Merge the key ranges of one (sequence, head).  A wavefront's lane l owns
// value dims 8l .. 8l+7.  Ranges go G at a time (G = 4, 8 or 16); the
// partial outputs, maxima and sums of a group are all requested before any
// is used, so a group costs one memory round trip.  A running maximum
// rescales what is already summed when a later group raises it (ranges
// without keys weigh zero).
constexpr int kCombineThreads = 256;
// The merge of up to 16 ranges runs one wavefront per workgroup: with few
// sequences its handful of wavefronts then spread over as many CUs (measured
// 0.4-0.6 us faster per call at 1 x 1024 and 8 x 512 keys than four per
// workgroup, and the same at 64 sequences).
constexpr int kNarrowThreads = 64;

// Ranges [s_begin, s_end) of one (sequence, head) into one wavefront's
// running (max M, weight sum den, weighted output acc over dims 8l .. 8l+7).
template <bool KVF8, int G>
__device__ __forceinline__ void combine_ranges(const Args& a, size_t p0, int s_begin, int s_end, int lane,
                                               float& M, float& den, f32x4& acc0, f32x4& acc1, float& kvs) {
    const float* po = a.part_o + p0 * kValue + 8 * lane;
    // s_end >= 1 and s_begin < s_end in both callers; a do-while has no
    // entry test, so the argument loads are not split by a wait for splits.
    int s0 = s_begin;
    do {
        f32x4 v[2 * G];
        float ms[G], ls[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int s = s0 + u < s_end ? s0 + u : s_end - 1;
            v[2 * u] = *reinterpret_cast<const f32x4*>(po + (size_t)s * kValue);
            v[2 * u + 1] = *reinterpret_cast<const f32x4*>(po + (size_t)s * kValue + 4);
            ms[u] = a.part_m[p0 + s];
            ls[u] = s0 + u < s_end ? a.part_l[p0 + s] : 0.0f;
        }
        if constexpr (KVF8) {
            // The scale is needed by the final store only.  Its load goes out
            // behind the first group's loads; the empty asm needs its value
            // here, so it is not deferred until after they return (a further
            // memory round trip before the store).
            if (s0 == s_begin) {
                kvs = *a.kv_scale;
                asm volatile("" ::"s"(kvs));
            }
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (ls[u] > 0.0f) Mn = fmaxf(Mn, ms[u]);
        if (Mn > M) {   // uniform: every lane reads the same maxima
            const float r = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
            acc0 *= r;
            acc1 *= r;
            den *= r;
            M = Mn;
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const float wgt = ls[u] > 0.0f ? __builtin_amdgcn_exp2f(ms[u] - M) : 0.0f;
            acc0 += wgt * v[2 * u];
            acc1 += wgt * v[2 * u + 1];
            den += wgt * ls[u];
        }
        s0 += G;
    } while (s0 < s_end);
}

template <bool KVF8>
__device__ __forceinline__ void combine_write(const Args& a, int bh, int lane, float den, f32x4 acc0, f32x4 acc1,
                                              float kvs) {
    float f = den > 0.0f ? 1.0f / den : 0.0f;
    if constexpr (KVF8) f *= kvs;
    uint16_t r[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = bf16_bits(acc0[e] * f);
        r[4 + e] = bf16_bits(acc1[e] * f);
    }
    u32x4 packed;
#pragma unroll
    for (int k = 0; k < 4; ++k) packed[k] = uint32_t(r[2 * k]) | (uint32_t(r[2 * k + 1]) << 16);
    *reinterpret_cast<u32x4*>(a.out + (size_t)bh * kValue + 8 * lane) = packed;
}

// Up to sixteen ranges: one wavefront per (sequence, head) and per workgroup.
template <bool KVF8, int G>
__global__ void __launch_bounds__(kNarrowThreads) mla_attn_combine_kernel(const Args a) {
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * (kNarrowThreads / 64) + (threadIdx.x >> 6);   // b * H + h
    // No early exit: a wavefront past the last head merges the last head
    // again and stores nothing, so the argument loads and the first partial
    // loads do not wait on a bounds test.
    const int nbh = a.B * a.H;                 // >= 1 whenever this kernel runs
    const int bhc = bh < nbh ? bh : nbh - 1;
    float M = -INFINITY, den = 0.0f, kvs = 1.0f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    combine_ranges<KVF8, G>(a, (size_t)bhc * a.splits, 0, a.splits, lane, M, den, acc0, acc1, kvs);
    if (bh < nbh) combine_write<KVF8>(a, bh, lane, den, acc0, acc1, kvs);
}

// More ranges: one workgroup per (sequence, head); its four wavefronts take
// a quarter of the ranges each and meet once in LDS.
template <bool KVF8>
__global__ void __launch_bounds__(kCombineThreads) mla_attn_combine_wide_kernel(const Args a) {
    __shared__ f32x4 part[kCombineThreads / 64][64][2];
    __shared__ float pm[kCombineThreads / 64][2];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    const int per = (a.splits + 3) / 4;
    const int sb = w * per < a.splits ? w * per : a.splits;
    const int se = sb + per < a.splits ? sb + per : a.splits;
    float M = -INFINITY, den = 0.0f, kvs = 1.0f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (per <= 8)
        combine_ranges<KVF8, 8>(a, (size_t)bh * a.splits, sb, se, lane, M, den, acc0, acc1, kvs);
    else
        combine_ranges<KVF8, 16>(a, (size_t)bh * a.splits, sb, se, lane, M, den, acc0, acc1, kvs);
    part[w][lane][0] = acc0;
    part[w][lane][1] = acc1;
    if (lane == 0) {
        pm[w][0] = M;
        pm[w][1] = den;
    }
    __syncthreads();
    if (w != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < kCombineThreads / 64; ++v)
        if (pm[v][1] > 0.0f) Mt = fmaxf(Mt, pm[v][0]);
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    float dt = 0.0f;
#pragma unroll
    for (int v = 0; v < kCombineThreads / 64; ++v) {
        const float wgt = pm[v][1] > 0.0f ? __builtin_amdgcn_exp2f(pm[v][0] - Mt) : 0.0f;
        t0 += wgt * part[v][lane][0];
        t1 += wgt * part[v][lane][1];
        dt += wgt * pm[v][1];
    }
    combine_write<KVF8>(a, bh, lane, dt, t0, t1, kvs);
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

// Workgroups the key split aims for (one resident per CU); the environment
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
    // at least one 64-key round per range (one tile per compute wavefront):
    // with few sequences, more and shorter ranges measured faster than
    // fewer, longer ones now that the merge takes many ranges per round trip
    const int64_t most = (steps + kMinSplitSteps - 1) / kMinSplitSteps;
    if (splits > most) splits = most;
    if (splits > kMaxSplits) splits = kMaxSplits;
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
    p->block_threads = ((flags & MLA_ATTN_KV_FP8) && kps > kStepKeys) ? kRingThreads : kThreads;
    return MLA_DQ_OK;
}

bool aligned(const void* x, uintptr_t n) { return (reinterpret_cast<uintptr_t>(x) % n) == 0; }

// Byte range [lo, lo + bytes) of one buffer; sizes saturate instead of wrapping.
struct Span {
    uintptr_t lo;
    uint64_t bytes;
};

uint64_t mul_sat(uint64_t a, uint64_t b) {
    uint64_t r;
    return __builtin_mul_overflow(a, b, &r) ? UINT64_MAX : r;
}

bool overlap(Span x, Span y) {
    if (x.bytes == 0 || y.bytes == 0) return false;
    const uint64_t xe = x.lo + x.bytes < x.lo ? UINT64_MAX : x.lo + x.bytes;
    const uint64_t ye = y.lo + y.bytes < y.lo ? UINT64_MAX : y.lo + y.bytes;
    return x.lo < ye && y.lo < xe;
}

// The output and the used part of the workspace are written while other
// workgroups still read the inputs, so neither may overlap any other buffer.
bool aliased(const void* out, const void* q, const void* cache, const int32_t* block_table,
             const int32_t* seq_lens, const float* q_scale, const float* kv_scale, const void* workspace,
             const mla_attn_dims* d, const mla_attn_plan& p, bool qf8, bool kvf8) {
    auto at = [](const void* x) { return reinterpret_cast<uintptr_t>(x); };
    const uint64_t bh = mul_sat(uint64_t(d->batch), uint64_t(d->num_heads));
    const Span o{at(out), mul_sat(bh, kValue * 2)};
    const Span ws{at(workspace), workspace ? uint64_t(p.workspace_bytes) : 0};
    const Span in[] = {
        {at(q), mul_sat(bh, qf8 ? kRow : 2 * kRow)},
        {at(cache), mul_sat(mul_sat(uint64_t(d->num_blocks), uint64_t(d->block_size)), kvf8 ? kRow : 2 * kRow)},
        {at(block_table), mul_sat(mul_sat(uint64_t(d->batch), uint64_t(d->max_blocks_per_seq)), 4)},
        {at(seq_lens), mul_sat(uint64_t(d->batch), 4)},
        {at(q_scale), qf8 ? 4u : 0u},
        {at(kv_scale), kvf8 ? 4u : 0u},
    };
    if (overlap(o, ws)) return true;
    for (const Span& s : in)
        if (overlap(o, s) || overlap(ws, s)) return true;
    return false;
}

template <bool QF8, bool KVF8>
hipError_t launch_pair(const Args& a, const mla_attn_plan& p, hipStream_t stream) {
    const dim3 grid(uint32_t(p.workgroups)), block(uint32_t(p.block_threads));
    const bool streamp = int64_t(a.B) * a.H * a.splits * kValue * 4 >= kStreamPartialBytes;
    if constexpr (KVF8) {
        if (a.keys_per_split == kStepKeys) {
            if (!p.combine) {
                hipLaunchKernelGGL((mla_attn_short_kernel<QF8, true, false>), grid, block, 0, stream, a);
                return hipGetLastError();
            }
            if (streamp)
                hipLaunchKernelGGL((mla_attn_short_kernel<QF8, false, true>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((mla_attn_short_kernel<QF8, false, false>), grid, block, 0, stream, a);
        } else {
            if (!p.combine) {
                hipLaunchKernelGGL((mla_attn_ring_kernel<QF8, true, false>), grid, block, 0, stream, a);
                return hipGetLastError();
            }
            if (streamp)
                hipLaunchKernelGGL((mla_attn_ring_kernel<QF8, false, true>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((mla_attn_ring_kernel<QF8, false, false>), grid, block, 0, stream, a);
        }
    } else {
        if (!p.combine) {
            hipLaunchKernelGGL((mla_attn_partial_kernel<QF8, true, false>), grid, block, 0, stream, a);
            return hipGetLastError();
        }
        if (streamp)
            hipLaunchKernelGGL((mla_attn_partial_kernel<QF8, false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((mla_attn_partial_kernel<QF8, false, false>), grid, block, 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t heads = uint32_t(a.B * a.H), per_block = kNarrowThreads / 64;
    const dim3 cgrid((heads + per_block - 1) / per_block), cblock(kNarrowThreads), wblock(kCombineThreads);
    if (a.splits <= 4)
        hipLaunchKernelGGL((mla_attn_combine_kernel<KVF8, 4>), cgrid, cblock, 0, stream, a);
    else if (a.splits <= 8)
        hipLaunchKernelGGL((mla_attn_combine_kernel<KVF8, 8>), cgrid, cblock, 0, stream, a);
    else if (a.splits <= 16)
        hipLaunchKernelGGL((mla_attn_combine_kernel<KVF8, 16>), cgrid, cblock, 0, stream, a);
    else
        hipLaunchKernelGGL((mla_attn_combine_wide_kernel<KVF8>), dim3(heads), wblock, 0, stream, a);
    return hipGetLastError();
}

// Scratch of mla_decode_attention_noalloc: the partial results of split key
// ranges for callers that cannot allocate or pass a workspace.  Every GPU
// the library runs on holds its own copy from the module's load until the
// process ends.  In host code this name is only a stand-in for the device
// symbol: kernels get the per-device address from scratch_address().
static __device__ __align__(256) uint8_t scratch[MLA_ATTN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the GPU that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current.  NULL if the lookup fails.
void* scratch_address(hipStream_t stream) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    static std::mutex lock;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> guard(lock);
    if (addr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

int attention(void* out, const void* q, const void* cache, const int32_t* block_table, const int32_t* seq_lens,
              const float* q_scale, const float* kv_scale, float sm_scale, void* workspace,
              size_t workspace_bytes, uint32_t flags, const mla_attn_dims* dims, hipStream_t stream,
              bool use_scratch) {
    mla_attn_plan p;
    int rc = make_plan(dims, flags, &p);
    if (rc != MLA_DQ_OK) return rc;
    if (dims->batch == 0) return MLA_DQ_OK;
    if (use_scratch && p.workspace_bytes > int64_t(MLA_ATTN_SCRATCH_BYTES)) return MLA_ATTN_ERR_SCRATCH;
    const bool qf8 = flags & MLA_ATTN_Q_FP8, kvf8 = flags & MLA_ATTN_KV_FP8;
    if (!out || !q || !cache || !block_table || !seq_lens) return MLA_DQ_ERR_NULL;
    if ((qf8 && !q_scale) || (kvf8 && !kv_scale)) return MLA_DQ_ERR_NULL;
    if (!use_scratch) {
        if (p.workspace_bytes > 0 && !workspace) return MLA_DQ_ERR_NULL;
        if (workspace_bytes < size_t(p.workspace_bytes)) return MLA_ATTN_ERR_WORKSPACE;
    }
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || (workspace && !aligned(workspace, 16)) ||
        (qf8 && !aligned(q_scale, 4)) || (kvf8 && !aligned(kv_scale, 4)))
        return MLA_DQ_ERR_ALIGN;
    if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return MLA_DQ_ERR_DIM;
    if (use_scratch) {
        // the library's own buffer, only where the split needs one
        workspace = p.workspace_bytes > 0 ? scratch_address(stream) : nullptr;
        if (p.workspace_bytes > 0 && workspace == nullptr) return MLA_DQ_ERR_LAUNCH;
    }
    if (aliased(out, q, cache, block_table, seq_lens, q_scale, kv_scale, workspace, dims, p, qf8, kvf8))
        return MLA_DQ_ERR_ALIAS;

    Args a;
    a.out = static_cast<uint16_t*>(out);
    a.q = static_cast<const uint8_t*>(q);
    a.cache = static_cast<const uint8_t*>(cache);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.q_scale = q_scale;
    a.kv_scale = kv_scale;
    const int64_t parts = dims->batch * dims->num_heads * int64_t(p.splits);
    a.part_o = p.workspace_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
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
    a.grid = int32_t(p.workgroups);
    hipError_t e;
    if (qf8)
        e = kvf8 ? launch_pair<true, true>(a, p, stream) : launch_pair<true, false>(a, p, stream);
    else
        e = kvf8 ? launch_pair<false, true>(a, p, stream) : launch_pair<false, false>(a, p, stream);
    return e == hipSuccess ? MLA_DQ_OK : MLA_DQ_ERR_LAUNCH;
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
    return mla_attn::attention(out, q, cache, block_table, seq_lens, q_scale, kv_scale, sm_scale, workspace,
                               workspace_bytes, flags, dims, static_cast<hipStream_t>(stream), false);
}

int mla_decode_attention_noalloc(void* out, const void* q, const void* cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const float* q_scale, const float* kv_scale,
                                 float sm_scale, uint32_t flags, const mla_attn_dims* dims, void* stream) {
    return mla_attn::attention(out, q, cache, block_table, seq_lens, q_scale, kv_scale, sm_scale, nullptr, 0,
                               flags, dims, static_cast<hipStream_t>(stream), true);
}

}  // extern "C"
