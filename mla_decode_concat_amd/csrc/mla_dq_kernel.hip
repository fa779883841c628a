// Fused MLA decode epilogue for gfx950 (MI355X).
//
// What it computes is defined in include/mla_dq.h (prhub summary of vLLM PR
// #54896, "Kimi-K3 MLA decode kernel": implementation breakdown items 1-3,
// key source snippets).  This file holds the device code and the launch.
//
// Work layout.  Every token owns H + 1 latent rows of 576 elements: its H
// query rows, then its cache row (the page's kernel orders a token's work
// items the same way: query slots first, then the cache slot).  A row is 72
// chunks of 8 elements -- 64 chunks of the 512-wide latent part, 8 chunks of
// the 64-wide positional tail -- and one chunk is one 16-byte bf16 load.
// Chunks are numbered flat, g = 72 * row + c, and every wavefront processes
// 64 consecutive chunks per step, starting at a multiple of 64.  Because
// 72 * row + 64 = 8 * row (mod 64), the 8 tail chunks of any row then sit in
// one aligned group of 8 lanes of one wavefront, and the NeoX partner of tail
// chunk j (element i pairs with i + 32, so chunk j with chunk j ^ 4) is lane
// (lane ^ 4): the rotation exchanges partner chunks with ds_swizzle, entirely
// in registers.
//
// Two mappings.  Small token counts are latency-bound (a few thousand
// chunks, far fewer than the chip has lanes), so each lane takes one chunk
// and every load is issued at once; a row spans 72 lanes, i.e. wavefronts per
// row.  Large token counts are bandwidth-bound, so each lane takes CPL chunks
// (loads for all of them in flight before the first store), i.e. rows per
// wavefront.  The page's kernel makes the same token-count-dependent choice
// with whole warps (implementation breakdown item 1); the threshold here is
// set by measurement on MI355X.
//
// Loads that do not depend on the upstream projection (slot, position, scale)
// are issued first, then the activations, then the rope table rows that need
// the position (the analogue of the page's reordering around its dependency
// wait, implementation breakdown item 2).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include "mla_dq.h"
#include "fastdiv.h"
#include "mla_dq_internal.h"

// Every product and sum of the rotation rounds on its own, like the
// reference definition: no contraction into fused multiply-adds.
#pragma clang fp contract(off)

namespace mla_dq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ void unpack_bf16(u32x4 d, float (&v)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        v[2 * p] = bf16_lo(d[p]);
        v[2 * p + 1] = bf16_hi(d[p]);
    }
}

template <int CPL, int BLOCK, bool ROPE, bool QF8, bool KVF8>
__global__ void __launch_bounds__(BLOCK)
mla_dq_epilogue_kernel(const KernelArgs a) {
    const uint32_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const uint32_t g0 = tile * uint32_t(CPL * BLOCK) + threadIdx.x;
    const uint32_t H = a.num_heads;

    // Per-chunk coordinates.
    uint32_t tok[CPL], head[CPL], chunk[CPL];
    bool live[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t g = g0 + uint32_t(k * BLOCK);
        live[k] = g < a.total_chunks;
        const uint32_t row = g / 72u;
        chunk[k] = g - row * 72u;
        tok[k] = fastdiv31(row, a.rows_per_token);
        head[k] = row - tok[k] * (H + 1);  // == H for the cache row
    }

    // Independent small loads first: scales, slots, positions.
    float q_inv = 1.0f, kv_inv = 1.0f;
    if constexpr (QF8) q_inv = 1.0f / *a.q_scale;
    if constexpr (KVF8) kv_inv = 1.0f / *a.kv_scale;
    int64_t slot[CPL];
    int64_t pos[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const bool is_cache = head[k] == H;
        slot[k] = (live[k] && is_cache) ? a.slot_mapping[tok[k]] : int64_t(-1);
        pos[k] = 0;
        if constexpr (ROPE) {
            if (live[k] && chunk[k] >= 64u) pos[k] = a.positions[tok[k]];
        }
    }

    // The activations: one 16-byte chunk per step.
    u32x4 d[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const bool is_cache = head[k] == H;
        const bool is_pe = chunk[k] >= 64u;
        const uint64_t t = tok[k];
        const uint16_t* src;
        if (!is_cache) {
            src = is_pe ? a.q_pe + t * a.q_pe_st + uint64_t(head[k]) * a.q_pe_sh + (chunk[k] - 64u) * 8u
                        : a.ql_nope + t * a.ql_nope_st + uint64_t(head[k]) * a.ql_nope_sh + chunk[k] * 8u;
        } else {
            src = is_pe ? a.k_pe + t * a.k_pe_st + (chunk[k] - 64u) * 8u
                        : a.kv_c + t * a.kv_c_st + chunk[k] * 8u;
        }
        d[k] = u32x4{0u, 0u, 0u, 0u};
        if (live[k]) d[k] = *reinterpret_cast<const u32x4*>(src);
    }

    // Rope table: tail chunk j needs cos and sin of angles 8*(j&3) .. +7.
    f32x4 cosv[ROPE ? CPL : 1][2], sinv[ROPE ? CPL : 1][2];
    if constexpr (ROPE) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            cosv[k][0] = cosv[k][1] = sinv[k][0] = sinv[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (live[k] && chunk[k] >= 64u) {
                int64_t p = pos[k];
                p = p < 0 ? 0 : (p >= a.max_position ? a.max_position - 1 : p);
                const float* row = a.rope_cos_sin + p * 64 + ((chunk[k] - 64u) & 3u) * 8u;
                cosv[k][0] = *reinterpret_cast<const f32x4*>(row);
                cosv[k][1] = *reinterpret_cast<const f32x4*>(row + 4);
                sinv[k][0] = *reinterpret_cast<const f32x4*>(row + 32);
                sinv[k][1] = *reinterpret_cast<const f32x4*>(row + 36);
            }
        }
    }

#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const bool is_cache = head[k] == H;
        const bool is_pe = chunk[k] >= 64u;
        float y[8];
        if constexpr (ROPE) {
            // Every lane takes part in the exchange; only tail lanes use it.
            const u32x4 partner = swap_lane4(d[k]);
            float own[8], par[8];
            unpack_bf16(d[k], own);
            unpack_bf16(partner, par);
            // First half (j < 4): y = x_i c - x_{i+32} s, own = x_i.
            // Second half:        y = x_{i+32} c + x_i s, own = x_{i+32}.
            const bool first = ((chunk[k] - 64u) & 4u) == 0u;
            const float c[8] = {cosv[k][0].x, cosv[k][0].y, cosv[k][0].z, cosv[k][0].w,
                                cosv[k][1].x, cosv[k][1].y, cosv[k][1].z, cosv[k][1].w};
            const float s[8] = {sinv[k][0].x, sinv[k][0].y, sinv[k][0].z, sinv[k][0].w,
                                sinv[k][1].x, sinv[k][1].y, sinv[k][1].z, sinv[k][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float oc = own[e] * c[e];
                const float ps = par[e] * s[e];
                y[e] = first ? oc - ps : oc + ps;
            }
        }
        if (!live[k]) continue;
        const bool rotated = ROPE && is_pe;
        const bool out_fp8 = is_cache ? KVF8 : QF8;
        uint8_t* dst;
        if (is_cache) {
            if (slot[k] < 0 || slot[k] >= a.num_slots) continue;
            dst = a.cache + (uint64_t(slot[k]) * 576u + chunk[k] * 8u) * (KVF8 ? 1u : 2u);
        } else {
            const uint64_t qrow = uint64_t(tok[k]) * H + head[k];
            dst = a.q_out + (qrow * 576u + chunk[k] * 8u) * (QF8 ? 1u : 2u);
        }
        if (out_fp8) {
            float v[8];
            if (rotated) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = y[e];
            } else {
                unpack_bf16(d[k], v);
            }
            *reinterpret_cast<u32x2*>(dst) = pack_e4m3(v, is_cache ? kv_inv : q_inv);
        } else {
            *reinterpret_cast<u32x4*>(dst) = rotated ? pack_bf16(y) : d[k];
        }
    }
}

template <int CPL, int BLOCK, bool ROPE, bool QF8, bool KVF8>
static hipError_t launch_one(const KernelArgs& a, uint32_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((mla_dq_epilogue_kernel<CPL, BLOCK, ROPE, QF8, KVF8>), dim3(grid),
                       dim3(BLOCK), 0, stream, a);
    return hipGetLastError();
}

template <int CPL, int BLOCK>
static hipError_t launch_flags(const KernelArgs& a, uint32_t grid, uint32_t flags,
                               hipStream_t stream) {
    const bool r = flags & MLA_DQ_ROPE, q = flags & MLA_DQ_Q_FP8, kv = flags & MLA_DQ_KV_FP8;
    if (r) {
        if (q) return kv ? launch_one<CPL, BLOCK, true, true, true>(a, grid, stream)
                         : launch_one<CPL, BLOCK, true, true, false>(a, grid, stream);
        return kv ? launch_one<CPL, BLOCK, true, false, true>(a, grid, stream)
                  : launch_one<CPL, BLOCK, true, false, false>(a, grid, stream);
    }
    if (q) return kv ? launch_one<CPL, BLOCK, false, true, true>(a, grid, stream)
                     : launch_one<CPL, BLOCK, false, true, false>(a, grid, stream);
    return kv ? launch_one<CPL, BLOCK, false, false, true>(a, grid, stream)
              : launch_one<CPL, BLOCK, false, false, false>(a, grid, stream);
}

hipError_t launch(const KernelArgs& a, const mla_dq_launch_plan& plan, uint32_t flags,
                  hipStream_t stream) {
    const uint32_t grid = (uint32_t)plan.grid_blocks;
    if (plan.mapping == 0)
        return launch_flags<kSmallCpl, kSmallBlock>(a, grid, flags, stream);
    return launch_flags<kLargeCpl, kLargeBlock>(a, grid, flags, stream);
}

}  // namespace mla_dq
