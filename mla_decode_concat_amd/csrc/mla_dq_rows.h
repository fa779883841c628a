// Device code of the fused MLA decode epilogue for gfx950 (MI355X): the
// workers that move latent parts and positional tails, shared by the epilogue
// kernel and by the epilogue fused into the W_UK product.
//
// What it computes is defined in include/mla_dq.h (prhub summary of vLLM PR
// #54896, "Kimi-K3 MLA decode kernel": implementation breakdown items 1-3,
// key source snippets).
//
// Work layout.  Every token owns H + 1 latent rows of 576 elements: its H
// query rows, then its cache row (the page's kernel orders a token's work
// items the same way: query slots first, then the cache slot).  A launch
// restricted to the query rows or to the cache rows enumerates only those
// (row_stride H or 1 rows per token).  A row is 72
// chunks of 8 bf16 elements, one chunk being one 16-byte load: 64 chunks of
// the 512-wide latent part and 8 chunks of the 64-wide positional tail.
//
//  * Latent parts.  64 chunks are exactly one 16-byte load per lane of a
//    wave64, so a wavefront moves one whole latent part per step.  The row,
//    and with it the token, head, slot and both base addresses, is uniform
//    across the wavefront and lives in scalar registers; each lane adds only
//    its own 16-byte offset.  Loads and stores are fully coalesced (1 KiB
//    contiguous per instruction), and the slot is a scalar load.
//  * Positional tails.  8 lanes take one row's 8 tail chunks, so a wavefront
//    takes the tails of 8 rows per step.  NeoX pairs element i with i + 32,
//    i.e. chunk j with chunk j ^ 4, which sits in lane (lane ^ 4): the
//    partner's 8 values arrive by ds_swizzle, in registers.  Each tail lane
//    takes the 8 cos and 8 sin values it needs from its token's table row:
//    in the throughput mapping the workgroup first stages the table rows of
//    its tokens in LDS (one 16-byte load per thread, then one barrier); in
//    the latency mapping, where that barrier would lengthen the critical
//    chain position -> table -> store, each lane loads its values itself.
//
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mla_dq.h"
#include "fastdiv.h"
#include "mla_dq_internal.h"

// Every product and sum of the rotation rounds on its own: no contraction
// into fused multiply-adds.
#pragma clang fp contract(off)

namespace mla_dq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Workgroup index -> tile index such that each of the 8 XCDs (which receive
// workgroups round-robin) works on one contiguous range of tiles.
__device__ __forceinline__ uint32_t xcd_contiguous_tile(uint32_t b, uint32_t n) {
    constexpr uint32_t kXcd = 8;
    const uint32_t per = n / kXcd, rem = n % kXcd;
    const uint32_t x = b % kXcd, i = b / kXcd;
    return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack_bf16(u32x4 d, float (&v)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        v[2 * p] = bf16_lo(d[p]);
        v[2 * p + 1] = bf16_hi(d[p]);
    }
}

// Eight activations (bf16 or fp16 bit patterns) -> eight exact fp32 values.
__device__ __forceinline__ void unpack_act(u32x4 d, float (&v)[8], bool fp16) {
    if (fp16) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            // through a scalar: a bit cast of the vector element expression
            // itself reads element 0 whatever p is
            const uint32_t word = d[p];
            const f16x2 h = __builtin_bit_cast(f16x2, word);
            v[2 * p] = (float)h.x;
            v[2 * p + 1] = (float)h.y;
        }
    } else {
        unpack_bf16(d, v);
    }
}

// Exchange a 16-byte chunk with lane (lane ^ 4) of the same wavefront.
__device__ __forceinline__ u32x4 swap_lane4(u32x4 v) {
    constexpr int kXor4 = 0x101F;  // ds_swizzle bit mode: and 0x1F, or 0, xor 4
    u32x4 r;
    r.x = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v.x, kXor4);
    r.y = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v.y, kXor4);
    r.z = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v.z, kXor4);
    r.w = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v.w, kXor4);
    return r;
}

// Clamp into the E4M3 range while keeping NaN a NaN.
__device__ __forceinline__ float clamp448(float v) {
    return __builtin_isnan(v) ? v : __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Eight fp32 values -> eight E4M3 codes (OCP format on gfx950, round to
// nearest even), value 0 in the lowest byte.
__device__ __forceinline__ u32x2 pack_e4m3(const float (&v)[8], float inv) {
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = clamp448(v[e] * inv);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[4], s[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[6], s[7], w1, true);
    u32x2 r;
    r.x = (uint32_t)w0;
    r.y = (uint32_t)w1;
    return r;
}

// Eight fp32 values -> eight bf16 (round to nearest even), value 0 lowest.
__device__ __forceinline__ u32x4 pack_bf16(const float (&v)[8]) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f32x2 f = {v[2 * p], v[2 * p + 1]};
        bf16x2 h = __builtin_convertvector(f, bf16x2);
        r[p] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

// Eight fp32 values -> eight fp16 (round to nearest even), value 0 lowest.
__device__ __forceinline__ u32x4 pack_f16(const float (&v)[8]) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f32x2 f = {v[2 * p], v[2 * p + 1]};
        f16x2 h = __builtin_convertvector(f, f16x2);
        r[p] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

template <bool STREAM, typename V>
__device__ __forceinline__ void store_out(uint8_t* p, V v) {
    if constexpr (STREAM)
        __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
    else
        *reinterpret_cast<V*>(p) = v;
}

template <bool STREAM, typename V>
__device__ __forceinline__ V load_in(const void* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
    else
        return *reinterpret_cast<const V*>(p);
}

// ---- latent parts: one 512-wide row per wavefront step ---------------------

// Raw buffer descriptor over [p, p + bytes): base, stride 0, num_records =
// bytes, and the GFX9-family word 3.  Accesses past num_records are dropped
// (stores) or return zero (loads) by the hardware, so a row that must not be
// read or written gets bytes = 0 instead of a branch.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x2 e4m3_of_act(u32x4 d, float inv, bool fp16) {
    float v[8];
    unpack_act(d, v, fp16);
    return pack_e4m3(v, inv);
}

template <int BLOCK, int RPW, bool STREAM, bool LF, bool VAR, bool QF8, bool KVF8>
__device__ __forceinline__ void latent_rows(const KernelArgs& a, uint32_t tile) {
    const bool fp16 = VAR && a.fp16;
    constexpr int kAux = STREAM ? MLA_DQ_STREAM_AUX : 0;
    constexpr uint32_t kWaves = BLOCK / kWave;
    constexpr uint32_t kQRowBytes = QF8 ? 576u : 1152u;
    constexpr uint32_t kKvRowBytes = KVF8 ? 576u : 1152u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t H = a.num_heads;
    const uint32_t row0 = tile * (kWaves * RPW) + wave;

    // Wave-uniform row coordinates (scalar registers).  Rows past the end
    // take row 0's coordinates and zero-sized descriptors.  The activation
    // loads go out first: they need nothing but the kernel arguments.
    uint32_t tok[RPW], head[RPW];
    bool live[RPW];
    u32x4 d[RPW];
    int64_t slot_early[RPW];
    float q_inv = 1.0f, kv_inv = 1.0f;
    if constexpr (!LF) {
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const uint32_t row = row0 + uint32_t(k) * kWaves;
            const uint32_t r = row < a.total_rows ? row : 0u;
            slot_early[k] = a.slot_mapping[fastdiv31(r, a.rows_per_token)];
        }
        if constexpr (QF8) q_inv = 1.0f / *a.q_scale;
        if constexpr (KVF8) kv_inv = 1.0f / *a.kv_scale;
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const uint32_t row = row0 + uint32_t(k) * kWaves;
        live[k] = row < a.total_rows;
        const uint32_t r = live[k] ? row : 0u;
        tok[k] = fastdiv31(r, a.rows_per_token);
        head[k] = r - tok[k] * a.row_stride + a.first_head;
        const uint16_t* sp = head[k] < H ? a.ql_nope + uint64_t(tok[k]) * a.ql_nope_st +
                                               uint64_t(head[k]) * a.ql_nope_sh
                                         : a.kv_c + uint64_t(tok[k]) * a.kv_c_st;
        d[k] = __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(sp, live[k] ? 1024u : 0u),
                                                     lane * 16u, 0, kAux);
    }
    // Slot and scales are needed by the stores only.
    if constexpr (LF) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QF8) q_inv = 1.0f / *a.q_scale;
        if constexpr (KVF8) kv_inv = 1.0f / *a.kv_scale;
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        const bool is_q = head[k] < H;
        const int64_t s = LF ? a.slot_mapping[tok[k]] : slot_early[k];
        const bool slot_ok = s >= 0 && s < a.num_slots;
        const __amdgpu_buffer_rsrc_t qdst =
            row_rsrc(a.q_out + (uint64_t(tok[k]) * H + head[k]) * kQRowBytes,
                     live[k] && is_q ? kQRowBytes : 0u);
        const __amdgpu_buffer_rsrc_t cdst =
            row_rsrc(a.cache + uint64_t(slot_ok ? s : 0) * kKvRowBytes,
                     live[k] && !is_q && slot_ok ? kKvRowBytes : 0u);
        // Each row is written through exactly one of its two descriptors; the
        // other has zero size, so that store is dropped.
        if constexpr (QF8 == KVF8) {
            const __amdgpu_buffer_rsrc_t dst = is_q ? qdst : cdst;
            if constexpr (QF8)
                __builtin_amdgcn_raw_buffer_store_b64(e4m3_of_act(d[k], is_q ? q_inv : kv_inv, fp16), dst,
                                                      lane * 8u, 0, kAux);
            else
                __builtin_amdgcn_raw_buffer_store_b128(d[k], dst, lane * 16u, 0, kAux);
        } else if constexpr (KVF8) {
            // Query rows copied, cache row E4M3.  The row is wave-uniform, so
            // a scalar branch spares the query rows (H of every H + 1) an
            // E4M3 conversion they would not store (measured 1.5 % faster at
            // 8192 tokens than converting every row).
            if (is_q)
                __builtin_amdgcn_raw_buffer_store_b128(d[k], qdst, lane * 16u, 0, kAux);
            else
                __builtin_amdgcn_raw_buffer_store_b64(e4m3_of_act(d[k], kv_inv, fp16), cdst, lane * 8u,
                                                      0, kAux);
        } else {
            // Query rows E4M3, cache row copied: the query rows convert
            // anyway, and issuing both stores (one dropped) measured faster
            // than branching.
            const u32x2 f8 = e4m3_of_act(d[k], q_inv, fp16);
            __builtin_amdgcn_raw_buffer_store_b64(f8, qdst, lane * 8u, 0, kAux);
            __builtin_amdgcn_raw_buffer_store_b128(d[k], cdst, lane * 16u, 0, kAux);
        }
    }
}

// ---- positional tails: 8 rows' tails per wavefront step --------------------
// Rows per workgroup of the tail worker, and the LDS it needs to stage
// their table rows (one 256-byte row per tail row at most).
template <int BLOCK, int STEPS>
constexpr uint32_t tail_table_lds_bytes() { return uint32_t(STEPS) * (BLOCK / 8) * 256u; }

// With TLDS, table_lds points to tail_table_lds_bytes<BLOCK, STEPS>() bytes of
// the workgroup's LDS (16-byte aligned), else it is unused.
template <int BLOCK, int STEPS, bool STREAM, bool LF, bool TLDS, bool VAR, bool ROPE, bool QF8, bool KVF8>
__device__ __forceinline__ void tail_rows(const KernelArgs& a, uint32_t tile, uint8_t* table_lds) {
    // Variant modes are read only by the instances built for them; the
    // page's configuration (bf16, NeoX pairs, fp32 table) checks nothing.
    const bool fp16 = VAR && a.fp16;
    const bool gptj = VAR && a.gptj;
    const bool table_bf16 = VAR && a.table_bf16;
    constexpr uint32_t kRowsPerStep = BLOCK / 8;
    const uint32_t H = a.num_heads;
    const uint32_t j = threadIdx.x % 8u;           // tail chunk 0..7
    const bool first_half = j < 4u;                // elements 8j..8j+7 < 32

    // Lanes past the last row read row 0 (always valid) and store nothing,
    // so every load below is unconditional.  Activations and positions go
    // first, then the table rows (which need the positions); slots and
    // scales are needed by the stores only.  With TLDS the positions are
    // read by the threads that stage the table rows, not by the tail lanes.
    uint32_t tok[STEPS], head[STEPS];
    bool live[STEPS];
    int64_t pos[STEPS], slot[STEPS];
    u32x4 d[STEPS];
    float q_inv = 1.0f, kv_inv = 1.0f;
    if constexpr (!LF) {
        if constexpr (QF8) q_inv = 1.0f / *a.q_scale;
        if constexpr (KVF8) kv_inv = 1.0f / *a.kv_scale;
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
            const uint32_t row = (tile * STEPS + k) * kRowsPerStep + threadIdx.x / 8u;
            const uint32_t r = row < a.total_rows ? row : 0u;
            slot[k] = a.slot_mapping[fastdiv31(r, a.rows_per_token)];
        }
    }
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        const uint32_t row = (tile * STEPS + k) * kRowsPerStep + threadIdx.x / 8u;
        live[k] = row < a.total_rows;
        const uint32_t r = live[k] ? row : 0u;
        tok[k] = fastdiv31(r, a.rows_per_token);
        head[k] = r - tok[k] * a.row_stride + a.first_head;
        const uint64_t t = tok[k];
        const uint16_t* src = head[k] < H
                                  ? a.q_pe + t * a.q_pe_st + uint64_t(head[k]) * a.q_pe_sh
                                  : a.k_pe + t * a.k_pe_st;
        d[k] = load_in<STREAM, u32x4>(src + j * 8u);
        pos[k] = 0;
        if constexpr (ROPE && !TLDS) pos[k] = a.positions[t];
    }
    // Table values for this lane, widened to one per element: cos in c, sin
    // in s.  NeoX: elements 8j..8j+7 of a half use angles 8(j&3)..+7.
    // Interleaved: elements 8j..8j+7 are pairs 4j..4j+3.
    float c[ROPE ? STEPS : 1][8], s[ROPE ? STEPS : 1][8];
    if constexpr (ROPE) {
        const uint32_t table_row_bytes = table_bf16 ? 128u : 256u;
        // TLDS: the workgroup's rows [rlo, rhi) belong to tokens t_lo ..
        // t_lo + ntok - 1.  Their table rows are copied to LDS, one 16-byte
        // chunk per thread, and every tail lane then reads its values there.
        // A token owns at least one row of the launch (one, when only cache
        // rows are written), so ntok <= rows.
        constexpr uint32_t kRowsPerWg = STEPS * kRowsPerStep;
        constexpr uint32_t kMaxTokens = kRowsPerWg;
        const uint8_t* staged = nullptr;
        uint32_t t_lo = 0;
        if constexpr (TLDS) {
            static_assert(kMaxTokens * 256u == tail_table_lds_bytes<BLOCK, STEPS>(), "table stage size");
            const uint32_t rlo = tile * kRowsPerWg;   // < total_rows: tile < tail_blocks
            const uint32_t rhi = rlo + kRowsPerWg < a.total_rows ? rlo + kRowsPerWg : a.total_rows;
            t_lo = fastdiv31(rlo, a.rows_per_token);
            const uint32_t ntok = fastdiv31(rhi - 1u, a.rows_per_token) - t_lo + 1u;
            const uint32_t shift = table_bf16 ? 3u : 4u;   // 16-byte chunks per row: 8 or 16
            for (uint32_t i = threadIdx.x; i < (ntok << shift); i += BLOCK) {
                const uint32_t k = i >> shift, q = i & ((1u << shift) - 1u);
                int64_t p = a.positions[t_lo + k];
                p = p < 0 ? 0 : (p >= a.max_position ? a.max_position - 1 : p);
                *reinterpret_cast<u32x4*>(table_lds + 256u * k + 16u * q) = *reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const uint8_t*>(a.rope_cos_sin) + p * table_row_bytes + 16u * q);
            }
            __syncthreads();
            staged = table_lds;
        }
#pragma unroll
        for (int k = 0; k < STEPS; ++k) {
            const uint8_t* row_base;
            if constexpr (TLDS) {
                row_base = staged + 256u * (live[k] ? tok[k] - t_lo : 0u);
            } else {
                int64_t p = pos[k];
                p = p < 0 ? 0 : (p >= a.max_position ? a.max_position - 1 : p);
                row_base = reinterpret_cast<const uint8_t*>(a.rope_cos_sin) + p * table_row_bytes;
            }
            const uint32_t col = gptj ? 4u * j : 8u * (j & 3u);
            if (table_bf16) {
                const uint16_t* trow = reinterpret_cast<const uint16_t*>(row_base) + col;
                if (gptj) {
                    const u32x2 cv = *reinterpret_cast<const u32x2*>(trow);
                    const u32x2 sv = *reinterpret_cast<const u32x2*>(trow + 32);
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        c[k][4 * q] = c[k][4 * q + 1] = bf16_lo(cv[q]);
                        c[k][4 * q + 2] = c[k][4 * q + 3] = bf16_hi(cv[q]);
                        s[k][4 * q] = s[k][4 * q + 1] = bf16_lo(sv[q]);
                        s[k][4 * q + 2] = s[k][4 * q + 3] = bf16_hi(sv[q]);
                    }
                } else {
                    unpack_bf16(*reinterpret_cast<const u32x4*>(trow), c[k]);
                    unpack_bf16(*reinterpret_cast<const u32x4*>(trow + 32), s[k]);
                }
            } else {
                const float* trow = reinterpret_cast<const float*>(row_base) + col;
                if (gptj) {
                    const f32x4 cv = *reinterpret_cast<const f32x4*>(trow);
                    const f32x4 sv = *reinterpret_cast<const f32x4*>(trow + 32);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c[k][2 * q] = c[k][2 * q + 1] = cv[q];
                        s[k][2 * q] = s[k][2 * q + 1] = sv[q];
                    }
                } else {
                    const f32x4 c0 = *reinterpret_cast<const f32x4*>(trow);
                    const f32x4 c1 = *reinterpret_cast<const f32x4*>(trow + 4);
                    const f32x4 s0 = *reinterpret_cast<const f32x4*>(trow + 32);
                    const f32x4 s1 = *reinterpret_cast<const f32x4*>(trow + 36);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c[k][q] = c0[q];
                        c[k][4 + q] = c1[q];
                        s[k][q] = s0[q];
                        s[k][4 + q] = s1[q];
                    }
                }
            }
        }
    }
    if constexpr (LF) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < STEPS; ++k) slot[k] = a.slot_mapping[tok[k]];
        // The scales are used only by the stores, behind a branch.  The
        // empty asm needs their values here, so their loads go out with the
        // table loads instead of being sunk past the wait for the table (a
        // third dependent memory round trip before the store).
        float qs = 1.0f, ks = 1.0f;
        if constexpr (QF8) qs = *a.q_scale;
        if constexpr (KVF8) ks = *a.kv_scale;
        asm volatile("" ::"s"(qs), "s"(ks));
        if constexpr (QF8) q_inv = 1.0f / qs;
        if constexpr (KVF8) kv_inv = 1.0f / ks;
    }
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        const bool is_q = head[k] < H;
        float y[8];
        if constexpr (ROPE) {
            // Each element e pairs with one partner: NeoX takes it from lane
            // (lane ^ 4) (chunk j ^ 4, every lane takes part in the exchange),
            // interleaved takes element e ^ 1 of the lane's own chunk.  The
            // first element of a pair gets own*c - partner*s, the second
            // own*c + partner*s.
            const u32x4 other = swap_lane4(d[k]);
            float own[8], par[8];
            unpack_act(d[k], own, fp16);
            if (gptj) {
#pragma unroll
                for (int e = 0; e < 8; ++e) par[e] = own[e ^ 1];
            } else {
                unpack_act(other, par, fp16);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool first = gptj ? (e & 1) == 0 : first_half;
                const float oc = own[e] * c[k][e];
                const float ps = par[e] * s[k][e];
                y[e] = first ? oc - ps : oc + ps;
            }
        } else {
            unpack_act(d[k], y, fp16);
        }
        const bool slot_ok = slot[k] >= 0 && slot[k] < a.num_slots;
        if (!live[k] || (!is_q && !slot_ok)) continue;
        const bool fp8 = is_q ? QF8 : KVF8;
        uint8_t* dst = is_q ? a.q_out + ((uint64_t(tok[k]) * H + head[k]) * 576u + 512u + j * 8u) *
                                            (QF8 ? 1u : 2u)
                            : a.cache + (uint64_t(slot[k]) * 576u + 512u + j * 8u) * (KVF8 ? 1u : 2u);
        if (fp8)
            store_out<STREAM>(dst, pack_e4m3(y, is_q ? q_inv : kv_inv));
        else if (ROPE)
            store_out<STREAM>(dst, fp16 ? pack_f16(y) : pack_bf16(y));
        else
            store_out<STREAM>(dst, d[k]);
    }
}

}  // namespace mla_dq
