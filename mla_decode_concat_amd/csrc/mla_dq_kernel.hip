// Fused MLA decode epilogue for gfx950 (MI355X): the kernel and its launch.
//
// What it computes is defined in include/mla_dq.h (prhub summary of vLLM PR
// #54896, "Kimi-K3 MLA decode kernel": implementation breakdown items 1-3,
// key source snippets).  The row workers and the work layout they follow are
// in mla_dq_rows.h.
//
// Workgroups [0, tail_blocks) do tails, the rest do latent parts; tails go
// first because their dependency chain (position -> table row -> rotate) is
// the longer one.
//
// Three mappings, chosen by the row count.  Small and mid token counts are
// latency-bound: every wavefront takes one latent row (and 8 tails), all
// loads are in flight at once, and the activations go out first; the small
// mapping uses one-wavefront workgroups, the mid mapping two-wavefront ones.
// Large token counts are bandwidth-bound: 256-thread workgroups batch two
// steps of tails per wavefront and stage the rope table rows in LDS.  The
// page's kernel makes the same token-count-dependent choice with whole warps
// (implementation breakdown item 1); the thresholds here are set by
// measurement on MI355X.
//
// Loads that do not depend on the upstream projection (slot, position,
// scale) are issued before the activations, as the page's kernel reorders
// its reads around the dependency wait (implementation breakdown item 2).
#include "mla_dq_rows.h"

namespace mla_dq {

template <int BLOCK, int RPW, int TAIL_STEPS, bool STREAM, bool VAR, bool ROPE, bool QF8, bool KVF8>
__global__ void __launch_bounds__(BLOCK)
mla_dq_epilogue_kernel(const KernelArgs a) {
    // The latency mappings (small-T and mid-T workgroup sizes) issue the
    // activation loads before anything the stores alone need; the throughput
    // mapping reads slots and scales first.
    constexpr bool kSmall = BLOCK != kLargeMapping.block;
    constexpr bool LATENT_LF = kSmall ? MLA_DQ_SMALL_LATENT_LF : MLA_DQ_LARGE_LATENT_LF;
    constexpr bool TAIL_LF = kSmall ? MLA_DQ_SMALL_TAIL_LF : MLA_DQ_LARGE_TAIL_LF;
    constexpr bool TABLE_LDS = kSmall ? MLA_DQ_SMALL_TABLE_LDS : MLA_DQ_LARGE_TABLE_LDS;
    const uint32_t b = blockIdx.x;
    if (b < a.tail_blocks) {
        if constexpr (TABLE_LDS) {
            __shared__ __attribute__((aligned(16))) uint8_t table_lds[tail_table_lds_bytes<BLOCK, TAIL_STEPS>()];
            tail_rows<BLOCK, TAIL_STEPS, STREAM, TAIL_LF, TABLE_LDS, VAR, ROPE, QF8, KVF8>(a, b, table_lds);
        } else {
            tail_rows<BLOCK, TAIL_STEPS, STREAM, TAIL_LF, TABLE_LDS, VAR, ROPE, QF8, KVF8>(a, b, nullptr);
        }
        return;
    }
    uint32_t tile = b - a.tail_blocks;
#if MLA_DQ_XCD_REMAP
    // tail_blocks is a multiple of 8, so tile and b share their XCD.
    tile = xcd_contiguous_tile(tile, gridDim.x - a.tail_blocks);
#endif
    latent_rows<BLOCK, RPW, STREAM, LATENT_LF, VAR, QF8, KVF8>(a, tile);
}

template <int BLOCK, int RPW, int TS, bool STREAM, bool VAR, bool ROPE, bool QF8, bool KVF8>
static hipError_t launch_one(const KernelArgs& a, uint32_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((mla_dq_epilogue_kernel<BLOCK, RPW, TS, STREAM, VAR, ROPE, QF8, KVF8>),
                       dim3(grid), dim3(BLOCK), 0, stream, a);
    return hipGetLastError();
}

template <int BLOCK, int RPW, int TS, bool STREAM, bool VAR>
static hipError_t launch_flags(const KernelArgs& a, uint32_t grid, uint32_t flags,
                               hipStream_t stream) {
    const bool r = flags & MLA_DQ_ROPE, q = flags & MLA_DQ_Q_FP8, kv = flags & MLA_DQ_KV_FP8;
    if (r) {
        if (q) return kv ? launch_one<BLOCK, RPW, TS, STREAM, VAR, true, true, true>(a, grid, stream)
                         : launch_one<BLOCK, RPW, TS, STREAM, VAR, true, true, false>(a, grid, stream);
        return kv ? launch_one<BLOCK, RPW, TS, STREAM, VAR, true, false, true>(a, grid, stream)
                  : launch_one<BLOCK, RPW, TS, STREAM, VAR, true, false, false>(a, grid, stream);
    }
    if (q) return kv ? launch_one<BLOCK, RPW, TS, STREAM, VAR, false, true, true>(a, grid, stream)
                     : launch_one<BLOCK, RPW, TS, STREAM, VAR, false, true, false>(a, grid, stream);
    return kv ? launch_one<BLOCK, RPW, TS, STREAM, VAR, false, false, true>(a, grid, stream)
              : launch_one<BLOCK, RPW, TS, STREAM, VAR, false, false, false>(a, grid, stream);
}

template <bool STREAM, bool VAR>
static hipError_t launch_mapping(const KernelArgs& a, const mla_dq_launch_plan& plan,
                                 uint32_t flags, hipStream_t stream) {
    const uint32_t grid = (uint32_t)plan.grid_blocks;
    if (plan.mapping == 0)
        return launch_flags<kSmallMapping.block, kSmallMapping.rows_per_wave,
                            kSmallMapping.tail_steps, STREAM, VAR>(a, grid, flags, stream);
    if (plan.mapping == 2)
        return launch_flags<kMidMapping.block, kMidMapping.rows_per_wave,
                            kMidMapping.tail_steps, STREAM, VAR>(a, grid, flags, stream);
    if constexpr (!STREAM) {
        if (plan.rows_per_wave == kMidSizeRowsPerWave && kMidSizeRowsPerWave != kLargeMapping.rows_per_wave)
            return launch_flags<kLargeMapping.block, kMidSizeRowsPerWave, kLargeMapping.tail_steps, STREAM, VAR>(
                a, grid, flags, stream);
    }
    return launch_flags<kLargeMapping.block, kLargeMapping.rows_per_wave,
                        kLargeMapping.tail_steps, STREAM, VAR>(a, grid, flags, stream);
}

hipError_t launch(const KernelArgs& a, const mla_dq_launch_plan& plan, uint32_t flags,
                  hipStream_t stream) {
    // Instances for the variant modes (fp16, interleaved pairs, bf16 table)
    // are separate, so that the page's configuration pays for none of them.
    const bool var = flags & (MLA_DQ_FP16 | MLA_DQ_ROPE_GPTJ | MLA_DQ_TABLE_BF16);
    if (plan.streaming)
        return var ? launch_mapping<true, true>(a, plan, flags, stream)
                   : launch_mapping<true, false>(a, plan, flags, stream);
    return var ? launch_mapping<false, true>(a, plan, flags, stream)
               : launch_mapping<false, false>(a, plan, flags, stream);
}

}  // namespace mla_dq
