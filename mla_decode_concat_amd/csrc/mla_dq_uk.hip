// The fused MLA decode epilogue inside the per-head W_UK product, for gfx950
// (MI355X).
//
// In a decode step the epilogue's ql_nope is the output of the absorbed key
// projection ql[t, h, :] = q_nope[t, h, 0:128] @ W_UK[h] ([128, 512] per
// head), and the page's kernel begins by waiting for that product
// (prhub summary of vLLM PR #54896, "implementation breakdown" item 2).  Here
// one launch does both: the product's result goes from the matrix cores'
// accumulators straight to its encoded q_out columns, so ql_nope never exists
// in memory.  The contract is in include/mla_dq.h.
//
// One grid, three kinds of workgroup (256 threads each):
//  * product workgroups [0, product_blocks): each takes one head h, one
//    group of latent columns and one range of tokens.  Its four wavefronts
//    each hold 16 * NB columns of W_UK[h] in registers, as operand A of
//    v_mfma_f32_16x16x32_{bf16,f16} (lane l: column n0 + 16b + l % 16, the
//    eight k = 32s + 8(l / 16) .. +7, read from w_uk_t, where k runs along
//    memory), and step through the token range 16 tokens at a time: operand
//    B is the 16 tokens' q_nope rows at the same k (the next step's rows are
//    loaded during this step's products), four products over k = 0..127
//    per 16-column block.  The result leaves lane l with token l % 16 and the
//    four consecutive columns 16b + 4(l / 16) .. +3, which it encodes and
//    stores (8 bytes bf16/fp16, 4 bytes E4M3).  Workgroups are dealt to the
//    eight XCDs round-robin; workgroup g takes column group g / 8 %
//    column_groups of its XCD's (g % 8) next unit, so the column groups that
//    read the same q_nope rows run back to back on one XCD and find them in
//    its L2.  From 64 heads each XCD takes a contiguous block of units in
//    head-major order (all token ranges of a head together: its W_UK
//    columns stay in that L2); with fewer heads unit 8 (g / 8 /
//    column_groups) + g % 8, ranges outermost, so that the XCDs read nearby
//    q_nope rows at the same time and each sees only the heads congruent to
//    its index modulo 8.
//  * tail workgroups: the positional tails of all T * (H + 1) rows, and
//  * cache workgroups: the latent parts of the T cache rows,
//    both done by the epilogue's own row workers (mla_dq_rows.h).
#include "mla_dq_rows.h"

namespace mla_dq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Operand type and matrix-core product of one activation type.
template <bool FP16>
struct Mfma {
    typedef bf16x8 operand;
    static __device__ __forceinline__ f32x4 run(operand a, operand b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<true> {
    typedef f16x8 operand;
    static __device__ __forceinline__ f32x4 run(operand a, operand b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Four fp32 values -> four bf16 or fp16 (round to nearest even), value 0 lowest.
template <bool FP16>
__device__ __forceinline__ u32x2 pack4_act(f32x4 v) {
    u32x2 r;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const f32x2 f = {v[2 * p], v[2 * p + 1]};
        if constexpr (FP16)
            r[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        else
            r[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    return r;
}

// Four fp32 values -> four E4M3 codes of fl32(v * inv) clamped to +-448
// (round to nearest even), value 0 in the lowest byte.
__device__ __forceinline__ uint32_t pack4_e4m3(f32x4 v, float inv) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[0] * inv), clamp448(v[1] * inv), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[2] * inv), clamp448(v[3] * inv), w, true);
    return uint32_t(w);
}

// s_waitcnt operand for "vector memory count 0", leaving the export and LDS /
// scalar counts at their maxima (no wait on them): vmcnt in bits 3:0 and
// 15:14, expcnt in 6:4, lgkmcnt in 11:8.
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __attribute__((address_space(3))) void lds_void;

// LDS of a staging product workgroup: the q_nope rows of its token range,
// then one output tile (16 tokens x the wavefront's columns) per wavefront.
template <int BLOCK, int NB, bool QF8>
constexpr uint32_t product_lds_bytes() {
    return MLA_DQ_UK_LARGE_TOKENS * 256u + uint32_t(BLOCK / kWave) * 16u * (16u * NB) * (QF8 ? 1u : 2u);
}

// One product workgroup (see the top of the file).  With STAGE (the
// throughput configuration) the token range's q_nope rows are staged in LDS
// and each step's results leave through a per-wavefront LDS tile as whole
// row segments; without it (the latency configuration) operands come
// straight from memory and results go straight out.  lds points to
// product_lds_bytes<BLOCK, NB, QF8>() bytes with STAGE.
template <int BLOCK, int NB, bool STAGE, bool STREAM, bool FP16, bool QF8>
__device__ __forceinline__ void product_tile(const UkArgs& u, uint32_t g, uint8_t* lds) {
    using Op = Mfma<FP16>;
    using V = typename Op::operand;
    constexpr uint32_t kWaves = BLOCK / kWave;
    constexpr uint32_t kCols = 16u * NB;                 // latent columns per wavefront
    constexpr uint32_t kOutBytes = QF8 ? 1u : 2u;
    constexpr uint32_t kRowBytes = 576u * kOutBytes;
    constexpr uint32_t kSegBytes = kCols * kOutBytes;    // one token's columns of this wavefront
    static_assert(512 % (kWaves * kCols) == 0, "column groups must tile the 512 latent columns");
    static_assert(kSegBytes % 16 == 0, "row segments are whole 16-byte chunks");
    // Without staging each store instruction writes 32 (or 16) bytes of 16
    // rows, which only the wavefront's next stores complete: non-temporal
    // stores of such partial lines measured far slower, so those stay cached
    // even when the rest of the call streams.
    constexpr bool kStreamStores = STREAM && (STAGE || MLA_DQ_UK_STREAM_PRODUCT_STORES);

    const uint32_t xcd = g % 8u, m = g / 8u;
    const uint32_t group = m % u.column_groups;
    const uint32_t H = u.tails.num_heads;
    uint32_t h, range;
    if (u.head_major) {
        const uint32_t pos = m / u.column_groups;        // place in this XCD's block of units
        const uint32_t unit = xcd * u.units_per_xcd + pos;
        if (pos >= u.units_per_xcd || unit >= u.units) return;   // whole workgroup: no barrier is skipped
        h = fastdiv31(unit, u.ranges);
        range = unit - h * u.ranges.div;
    } else {
        const uint32_t unit = 8u * (m / u.column_groups) + xcd;
        if (unit >= u.units) return;                      // whole workgroup: no barrier is skipped
        range = fastdiv31(unit, u.heads);
        h = unit - range * H;
    }
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t c = lane % 16u, kq = lane / 16u;
    const uint32_t n0 = (group * kWaves + wave) * kCols;

    // Operand A: W_UK[h][k][n] for this lane's column n and k slice, i.e.
    // 16 bytes of row n of w_uk_t[h].
    V wa[NB][4];
    const uint16_t* wrow = u.w_uk_t + (uint64_t(h) * 512u + n0 + c) * 128u + 8u * kq;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            wa[b][s] = __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(wrow + b * 16 * 128 + 32 * s));

    float inv = 1.0f;
    if constexpr (QF8) inv = 1.0f / *u.tails.q_scale;
    const uint32_t T = u.num_tokens;
    const uint32_t t_begin = range * u.tokens_per_group;
    const uint32_t t_end = T - t_begin < u.tokens_per_group ? T : t_begin + u.tokens_per_group;
    uint8_t* const q_out = u.tails.q_out;

    // The 16 x (16 NB) products of the 16 tokens from t0 (operand B: qv),
    // four matrix-core products over k per 16-column block.  Lane (c, kq)
    // ends with token c's columns 16b + 4kq .. +3 in acc[b].
    auto product = [&](const V (&qv)[4], f32x4 (&acc)[NB]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = Op::run(wa[b][s], qv[s], acc[b]);
    };

    if constexpr (STAGE) {
        // The range's q_nope rows go to LDS first, all loads in flight at
        // once (one 1 KiB direct-to-LDS load per four rows, the workgroup's
        // wavefronts taking turns), and every step then reads its operands
        // there.  Row r's 16-byte chunk j sits in slot j ^ (r % 16), so the
        // 16 rows one operand read covers hit 16 different bank groups.
        constexpr uint32_t kMaxTokens = MLA_DQ_UK_LARGE_TOKENS;
        static_assert((kMaxTokens & (kMaxTokens - 1)) == 0, "the staged range wraps with a mask");
        uint8_t* const q_lds = lds;
        // This wavefront's output tile: token r's segment at r * kSegBytes,
        // its 16-byte chunk j in slot j ^ (r % kChunks) (the reads below
        // then cover every bank once).
        uint8_t* const o_lds = lds + kMaxTokens * 256u + wave * 16u * kSegBytes;
        constexpr uint32_t kChunks = kSegBytes / 16u;        // chunks per token segment
        constexpr uint32_t kTokensPerRead = 64u / kChunks;
        constexpr uint32_t kReads = (16u + kTokensPerRead - 1u) / kTokensPerRead;

        const uint32_t rows = t_end - t_begin;               // <= tokens_per_group <= kMaxTokens
        const uint32_t loads = (rows + 3u) / 4u;
        const uint16_t* qhead = u.q_nope + uint64_t(h) * u.q_nope_sh;
        for (uint32_t i = wave; i < loads; i += kWaves) {
            const uint32_t r = 4u * i + lane / 16u;
            const uint32_t t = t_begin + r < T ? t_begin + r : T - 1u;
            const uint32_t j = (lane % 16u) ^ (r % 16u);
            __builtin_amdgcn_global_load_lds(qhead + uint64_t(t) * u.q_nope_st + 8u * j,
                                             (lds_void*)(q_lds + 1024u * i), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the weights and this wavefront's rows
        __syncthreads();                            // everyone's rows

        // Operands of the 16 rows from r0 (modulo the stage, so that the
        // look-ahead past the last step stays inside it).
        auto read_rows = [&](uint32_t r0, V (&qv)[4]) {
            const uint8_t* row = q_lds + ((r0 + c) & (kMaxTokens - 1u)) * 256u;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qv[s] = __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(row + 16u * ((4u * s + kq) ^ c)));
        };
        // Products, encoding into the output tile, then whole segments out:
        // token r's 16-byte chunk j goes to its row at column n0 + 16 j / out
        // bytes, kChunks lanes per token (128 or 64 contiguous bytes).
        auto step = [&](const V (&qv)[4], uint32_t r0) {
            f32x4 acc[NB];
            product(qv, acc);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if constexpr (QF8) {
                    const uint32_t slot = (uint32_t(b) ^ (c % kChunks)) * 16u + 4u * kq;
                    *reinterpret_cast<uint32_t*>(o_lds + c * kSegBytes + slot) = pack4_e4m3(acc[b], inv);
                } else {
                    const uint32_t slot = ((2u * b + kq / 2u) ^ (c % kChunks)) * 16u + 8u * (kq & 1u);
                    *reinterpret_cast<u32x2*>(o_lds + c * kSegBytes + slot) = pack4_act<FP16>(acc[b]);
                }
            }
#pragma unroll
            for (uint32_t rd = 0; rd < kReads; ++rd) {
                const uint32_t r = rd * kTokensPerRead + lane / kChunks, j = lane % kChunks;
                const uint32_t t = t_begin + r0 + r;
                const u32x4 v = *reinterpret_cast<const u32x4*>(o_lds + (r % 16u) * kSegBytes + ((j ^ (r % kChunks)) * 16u));
                if (r < 16u && t < t_end)
                    store_out<kStreamStores>(q_out + (uint64_t(t) * H + h) * kRowBytes + n0 * kOutBytes + 16u * j, v);
            }
        };
        // Two operand buffers in turn: the next step's reads go out before
        // this step's products.
        V qa[4], qb[4];
        read_rows(0, qa);
        const uint32_t steps = (rows + 15u) / 16u;
        uint32_t r0 = 0;
        for (uint32_t i = 1; i < steps; i += 2, r0 += 32u) {
            read_rows(r0 + 16u, qb);
            __builtin_amdgcn_sched_barrier(0);
            step(qa, r0);
            read_rows(r0 + 32u, qa);
            __builtin_amdgcn_sched_barrier(0);
            step(qb, r0 + 16u);
        }
        if (steps & 1u) step(qa, r0);
    } else {
        const uint16_t* qcol = u.q_nope + uint64_t(h) * u.q_nope_sh + 8u * kq;
        // Operand B: 16 bytes of token t's q_nope row; lanes past the last
        // token read the last token's row (always valid) and store nothing.
        auto load_tokens = [&](uint32_t t0, V (&qv)[4]) {
            const uint32_t t = t0 + c < T ? t0 + c : T - 1u;
            const uint16_t* p = qcol + uint64_t(t) * u.q_nope_st;
#pragma unroll
            for (int s = 0; s < 4; ++s) qv[s] = __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(p + 32 * s));
        };
        auto step = [&](const V (&qv)[4], uint32_t t0) {
            f32x4 acc[NB];
            product(qv, acc);
            const uint32_t t = t0 + c;
            if (t < t_end) {
                uint8_t* dst = q_out + (uint64_t(t) * H + h) * kRowBytes + (n0 + 4u * kq) * kOutBytes;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if constexpr (QF8)
                        store_out<kStreamStores>(dst + 16u * b, pack4_e4m3(acc[b], inv));
                    else
                        store_out<kStreamStores>(dst + 32u * b, pack4_act<FP16>(acc[b]));
                }
            }
        };
        // Two operand buffers in turn, the next step's rows loading from
        // memory while this step's products run (a copy between buffers
        // would wait for them).  The weights and the first rows are waited
        // for in full before the loop, so that its waits cover only what the
        // loop itself issues; the loop runs whole pairs of steps and leaves
        // only at its end (an exit between the two halves would let the
        // unused look-ahead load reach the loop top, which then waits for
        // everything), an odd last step follows it.  The scheduling barriers
        // keep each look-ahead load ahead of the products it overlaps.
        // Look-ahead loads past the range read clamped, valid rows.
        V qa[4], qb[4];
        load_tokens(t_begin, qa);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const uint32_t steps = (t_end - t_begin + 15u) / 16u;
        uint32_t t0 = t_begin;
        for (uint32_t i = 1; i < steps; i += 2, t0 += 32u) {
            load_tokens(t0 + 16u, qb);
            __builtin_amdgcn_sched_barrier(0);
            step(qa, t0);
            load_tokens(t0 + 32u, qa);
            __builtin_amdgcn_sched_barrier(0);
            step(qb, t0 + 16u);
        }
        if (steps & 1u) step(qa, t0);
    }
}

}  // namespace

template <int NB, int TAIL_STEPS, bool LARGE, bool STREAM, bool VAR, bool ROPE, bool QF8, bool KVF8>
__global__ void __launch_bounds__(MLA_DQ_UK_BLOCK)
mla_dq_uk_epilogue_kernel(const UkArgs u) {
    constexpr int kBlock = MLA_DQ_UK_BLOCK;
    constexpr bool LATENT_LF = LARGE ? MLA_DQ_LARGE_LATENT_LF : MLA_DQ_SMALL_LATENT_LF;
    constexpr bool TAIL_LF = LARGE ? MLA_DQ_LARGE_TAIL_LF : MLA_DQ_SMALL_TAIL_LF;
    constexpr bool TABLE_LDS = LARGE ? MLA_DQ_LARGE_TABLE_LDS : MLA_DQ_SMALL_TABLE_LDS;
    // One LDS block serves whichever kind of work the workgroup does.
    constexpr uint32_t kTable = TABLE_LDS ? tail_table_lds_bytes<kBlock, TAIL_STEPS>() : 0u;
    constexpr uint32_t kProduct = LARGE ? product_lds_bytes<kBlock, NB, QF8>() : 0u;
    constexpr uint32_t kBoth = kTable > kProduct ? kTable : kProduct;
    constexpr uint32_t kLds = kBoth > 16u ? kBoth : 16u;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
    uint32_t b = blockIdx.x;
    if (b < u.product_blocks) {
        if (VAR && u.tails.fp16)
            product_tile<kBlock, NB, LARGE, STREAM, true, QF8>(u, b, lds);
        else
            product_tile<kBlock, NB, LARGE, STREAM, false, QF8>(u, b, lds);
        return;
    }
    b -= u.product_blocks;
    if (b < u.tail_blocks) {
        tail_rows<kBlock, TAIL_STEPS, STREAM, TAIL_LF, TABLE_LDS, VAR, ROPE, QF8, KVF8>(u.tails, b, lds);
        return;
    }
    latent_rows<kBlock, 1, STREAM, LATENT_LF, VAR, QF8, KVF8>(u.cache_rows, b - u.tail_blocks);
}

namespace {

template <int NB, int TS, bool LARGE, bool STREAM, bool VAR, bool ROPE, bool QF8, bool KVF8>
hipError_t uk_one(const UkArgs& u, uint32_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((mla_dq_uk_epilogue_kernel<NB, TS, LARGE, STREAM, VAR, ROPE, QF8, KVF8>), dim3(grid),
                       dim3(MLA_DQ_UK_BLOCK), 0, stream, u);
    return hipGetLastError();
}

template <int NB, int TS, bool LARGE, bool STREAM, bool VAR>
hipError_t uk_flags(const UkArgs& u, uint32_t grid, uint32_t flags, hipStream_t stream) {
    const bool r = flags & MLA_DQ_ROPE, q = flags & MLA_DQ_Q_FP8, kv = flags & MLA_DQ_KV_FP8;
    if (r) {
        if (q) return kv ? uk_one<NB, TS, LARGE, STREAM, VAR, true, true, true>(u, grid, stream)
                         : uk_one<NB, TS, LARGE, STREAM, VAR, true, true, false>(u, grid, stream);
        return kv ? uk_one<NB, TS, LARGE, STREAM, VAR, true, false, true>(u, grid, stream)
                  : uk_one<NB, TS, LARGE, STREAM, VAR, true, false, false>(u, grid, stream);
    }
    if (q) return kv ? uk_one<NB, TS, LARGE, STREAM, VAR, false, true, true>(u, grid, stream)
                     : uk_one<NB, TS, LARGE, STREAM, VAR, false, true, false>(u, grid, stream);
    return kv ? uk_one<NB, TS, LARGE, STREAM, VAR, false, false, true>(u, grid, stream)
              : uk_one<NB, TS, LARGE, STREAM, VAR, false, false, false>(u, grid, stream);
}

template <bool STREAM, bool VAR>
hipError_t uk_config(const UkArgs& u, const mla_dq_uk_launch_plan& p, uint32_t flags, hipStream_t stream) {
    const uint32_t grid = uint32_t(p.grid_blocks);
    if (p.mapping == 1) {
        if (p.n_blocks == 2) return uk_flags<2, kLargeMapping.tail_steps, true, STREAM, VAR>(u, grid, flags, stream);
        return uk_flags<MLA_DQ_UK_LARGE_NB, kLargeMapping.tail_steps, true, STREAM, VAR>(u, grid, flags, stream);
    }
    if (p.n_blocks == 1) return uk_flags<1, 1, false, STREAM, VAR>(u, grid, flags, stream);
    return uk_flags<MLA_DQ_UK_SMALL_NB, 1, false, STREAM, VAR>(u, grid, flags, stream);
}

}  // namespace

hipError_t launch_uk(const UkArgs& u, const mla_dq_uk_launch_plan& p, uint32_t flags, hipStream_t stream) {
    const bool var = flags & (MLA_DQ_FP16 | MLA_DQ_ROPE_GPTJ | MLA_DQ_TABLE_BF16);
    if (p.streaming)
        return var ? uk_config<true, true>(u, p, flags, stream) : uk_config<true, false>(u, p, flags, stream);
    return var ? uk_config<false, true>(u, p, flags, stream) : uk_config<false, false>(u, p, flags, stream);
}

}  // namespace mla_dq
