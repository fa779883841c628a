// Internal declarations shared by the launch code and the kernel file.
#pragma once

#include <stdint.h>

#include "mla_dq.h"
#include "fastdiv.h"

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#endif

// Tuning knobs (compile-time; the defaults are the measured choice on
// MI355X).  Workgroup sizes, latent rows per wavefront and tail steps of the
// two mappings, and the default thresholds of the launch plan.
#ifndef MLA_DQ_SMALL_BLOCK
#define MLA_DQ_SMALL_BLOCK 64
#endif
#ifndef MLA_DQ_MID_BLOCK
#define MLA_DQ_MID_BLOCK 128
#endif
#ifndef MLA_DQ_LARGE_BLOCK
#define MLA_DQ_LARGE_BLOCK 256
#endif
#ifndef MLA_DQ_LARGE_ROWS_PER_WAVE
#define MLA_DQ_LARGE_ROWS_PER_WAVE 1
#endif
// Latent rows per wavefront of the throughput mapping for mid-size calls
// under the default cache policy (bytes in [MIN, MAX]): two rows in flight per
// wavefront measured 2-8 % faster from 28 to 86 MB at 128 heads and at 40 MB
// at 16 heads, and slower on larger calls whose data is not yet in cache.
#ifndef MLA_DQ_MID_SIZE_ROWS_PER_WAVE
#define MLA_DQ_MID_SIZE_ROWS_PER_WAVE 2
#endif
#ifndef MLA_DQ_MID_SIZE_BYTES_MIN
#define MLA_DQ_MID_SIZE_BYTES_MIN (24ll << 20)
#endif
#ifndef MLA_DQ_MID_SIZE_BYTES_MAX
#define MLA_DQ_MID_SIZE_BYTES_MAX (96ll << 20)
#endif
#ifndef MLA_DQ_LARGE_TAIL_STEPS
#define MLA_DQ_LARGE_TAIL_STEPS 2
#endif
// Small-T mapping while T * (H + 1) <= the first threshold, mid-T mapping
// (the same latency settings in 128-thread workgroups) up to the second,
// throughput mapping above.  Measured on MI355X for 16 to 128 heads, with
// the epilogue right after the per-head W_UK product of a decode step (its
// place in a model): the 64-thread workgroups win up to about 900 rows, and
// with at most 32 heads up to about 2600 rows; the 128-thread ones up to
// about 5000 to 6000.
#ifndef MLA_DQ_SMALL_ROWS_MAX_DEFAULT
#define MLA_DQ_SMALL_ROWS_MAX_DEFAULT 896
#endif
#ifndef MLA_DQ_SMALL_ROWS_MAX_FEW_HEADS_DEFAULT
#define MLA_DQ_SMALL_ROWS_MAX_FEW_HEADS_DEFAULT 2560
#endif
#ifndef MLA_DQ_FEW_HEADS_MAX
#define MLA_DQ_FEW_HEADS_MAX 32
#endif
#ifndef MLA_DQ_MID_ROWS_MAX_DEFAULT
#define MLA_DQ_MID_ROWS_MAX_DEFAULT 5120
#endif
// Streaming (non-temporal) loads and stores once a call moves at least this
// many bytes.  Measured inside a captured decode step (the producing GEMMs
// before the call; graph-replayed, nine alternating rounds), both the
// epilogue and the fused W_UK call gain from streaming from about 85 MB on
// (epilogue at 102 / 117 / 146 MB: 22.3-26.5 -> 18.5, 26.1-27.9 -> 22.3,
// 32.1 -> 28.3 us; fused call at 91 / 100 MB: 32.5 -> 29.2, 37.0 -> 31.3 us)
// and lose or break even below (epilogue at 73 MB 13.1 -> 13.8 us, fused
// call at 73 MB 23.8 -> 24.5 us).  A call replayed alone on one resident
// buffer set would keep the cached policy up to the 256 MB Infinity Cache
// (2-7 % faster there), but in a step the neighbouring kernels' data leave
// little of it resident.
#ifndef MLA_DQ_STREAM_BYTES_MIN_DEFAULT
#define MLA_DQ_STREAM_BYTES_MIN_DEFAULT (80ll << 20)
#endif
// Cache-policy bits for streaming buffer loads and stores (the non-temporal
// bit of gfx94x/gfx950).
#ifndef MLA_DQ_STREAM_AUX
#define MLA_DQ_STREAM_AUX 2
#endif
// Deal each XCD one contiguous range of latent workgroups (measured slower
// for this streaming kernel, so off).
#ifndef MLA_DQ_XCD_REMAP
#define MLA_DQ_XCD_REMAP 0
#endif

// Load order per mapping and workgroup kind: 1 = activations (and
// positions) first, slots and scales after them; 0 = slots and scales first.
#ifndef MLA_DQ_SMALL_LATENT_LF
#define MLA_DQ_SMALL_LATENT_LF 1
#endif
#ifndef MLA_DQ_SMALL_TAIL_LF
#define MLA_DQ_SMALL_TAIL_LF 1
#endif
#ifndef MLA_DQ_LARGE_LATENT_LF
#define MLA_DQ_LARGE_LATENT_LF 0
#endif
#ifndef MLA_DQ_LARGE_TAIL_LF
#define MLA_DQ_LARGE_TAIL_LF 0
#endif

// Where tail lanes read the rope table: 1 = the workgroup first stages the
// table rows of its tokens in LDS, 0 = each lane loads its own values from
// the table.  Staging saves table loads and costs one barrier: it wins when
// bandwidth-bound and loses on the latency-bound path (measured).
#ifndef MLA_DQ_SMALL_TABLE_LDS
#define MLA_DQ_SMALL_TABLE_LDS 0
#endif
#ifndef MLA_DQ_LARGE_TABLE_LDS
#define MLA_DQ_LARGE_TABLE_LDS 1
#endif

// The epilogue fused into the W_UK product: workgroup size, 16-column
// blocks of W_UK per wavefront and tokens per product workgroup of its two
// configurations, and the query-row count T * H from which the throughput
// configuration is the default.
#ifndef MLA_DQ_UK_BLOCK
#define MLA_DQ_UK_BLOCK 256
#endif
#ifndef MLA_DQ_UK_SMALL_NB
#define MLA_DQ_UK_SMALL_NB 2
#endif
// The latency configuration takes one 16-column block per wavefront instead
// (twice the product workgroups, each loading half the weight columns) while
// it has at most this many (head, token range) units: measured at 16 heads,
// 1 / 16 / 32 tokens 3.05 -> 2.55, 3.44 -> 2.95, 3.49 -> 3.15 us; at 48
// tokens (48 units) 3.51 -> 3.83, and at 128 heads slower from one token.
#ifndef MLA_DQ_UK_SMALL_NB1_UNITS_MAX
#define MLA_DQ_UK_SMALL_NB1_UNITS_MAX 32
#endif
#ifndef MLA_DQ_UK_SMALL_TOKENS
#define MLA_DQ_UK_SMALL_TOKENS 16
#endif
#ifndef MLA_DQ_UK_LARGE_NB
#define MLA_DQ_UK_LARGE_NB 4
#endif
#ifndef MLA_DQ_UK_LARGE_TOKENS
#define MLA_DQ_UK_LARGE_TOKENS 128
#endif
// The throughput configuration takes two 16-column blocks per wavefront
// instead of MLA_DQ_UK_LARGE_NB up to this many query rows T * H, from this
// many tokens: twice the column groups, so that each product workgroup
// loops over half the columns of its tokens.  With fewer tokens per head the
// extra workgroups only add weight loads.  Measured (graph replays, E4M3 q):
// 65 / 128 / 192 / 1024 tokens x 16 heads 4.19 -> 4.06, 4.75 -> 4.00,
// 6.08 -> 4.64, 8.64 -> 8.27 us; 64 / 128 tokens x 128 heads 6.44 -> 6.37,
// 9.05 -> 8.82 us; slower at 9-48 tokens x 128 heads (5.17 -> 5.26 at 9,
// 5.92 -> 6.06 at 48) and from 32768 rows (2048 x 16: 12.96 -> 13.37 us,
// 256 x 128: 12.88 -> 13.43 us).
#ifndef MLA_DQ_UK_LARGE_NB2_ROWS_MAX
#define MLA_DQ_UK_LARGE_NB2_ROWS_MAX 16384
#endif
#ifndef MLA_DQ_UK_LARGE_NB2_TOKENS_MIN
#define MLA_DQ_UK_LARGE_NB2_TOKENS_MIN 64
#endif
// 1 = the latency configuration's product stores also stream when the call
// streams (they write partial lines, measured far slower that way).
#ifndef MLA_DQ_UK_STREAM_PRODUCT_STORES
#define MLA_DQ_UK_STREAM_PRODUCT_STORES 0
#endif
// The throughput configuration halves its tokens per product workgroup
// (down to 16) while fewer than this many product workgroups would result:
// one per CU.  Every product workgroup loads its columns of W_UK (64 KiB),
// so shorter token ranges mostly add weight reads; measured against 2048 (and
// 1024, 512, 128, 64): 1024 x 16 tokens 18.4 -> 8.7 us, 256 x 128 heads
// 20.5 -> 13.3 us, 256 x 16 6.7 -> 5.1 us, 8192 x 16 unchanged.
// Order of the product units from this many heads on: head-major, each
// XCD taking a contiguous block of ceil(units / 8) units (all token ranges
// of its heads back to back, so that their W_UK columns stay in its L2);
// below it range-major, unit u dealt to XCD u % 8 (the XCDs then work on the
// same token range at once, which keeps their q_nope reads close together).
#ifndef MLA_DQ_UK_HEAD_MAJOR_HEADS_MIN
#define MLA_DQ_UK_HEAD_MAJOR_HEADS_MIN 64
#endif
#ifndef MLA_DQ_UK_TARGET_BLOCKS
#define MLA_DQ_UK_TARGET_BLOCKS 256
#endif
// The same for the latency configuration.
#ifndef MLA_DQ_UK_SMALL_TARGET_BLOCKS
#define MLA_DQ_UK_SMALL_TARGET_BLOCKS 256
#endif
// Measured crossover (graph replays, 16 and 128 heads): the latency
// configuration wins up to 1024 query rows (64 x 16: 3.6 against 4.2 us;
// 8 x 128 equal), the throughput one past them (65 x 16: 4.2 against 4.5
// us, a fifth 16-token range per head then costing the latency one more
// than one product workgroup per CU; 72 x 16: 4.2 against 4.6 us).
#ifndef MLA_DQ_UK_LARGE_ROWS_MIN_DEFAULT
#define MLA_DQ_UK_LARGE_ROWS_MIN_DEFAULT 1025
#endif

namespace mla_dq {

// A mapping: threads per workgroup, latent rows handled by each wavefront
// (one row = 64 chunks = one 16-byte load per lane), and steps of 8 tails
// per wavefront for the positional part.
struct Mapping {
    int block;
    int rows_per_wave;
    int tail_steps;
};
constexpr Mapping kSmallMapping{MLA_DQ_SMALL_BLOCK, 1, 1};
constexpr Mapping kMidMapping{MLA_DQ_MID_BLOCK, 1, 1};
constexpr Mapping kLargeMapping{MLA_DQ_LARGE_BLOCK, MLA_DQ_LARGE_ROWS_PER_WAVE,
                                MLA_DQ_LARGE_TAIL_STEPS};
// The kernel tells the latency mappings from the throughput mapping by the
// workgroup size.
static_assert(kSmallMapping.block != kLargeMapping.block && kMidMapping.block != kLargeMapping.block &&
                  kSmallMapping.block != kMidMapping.block,
              "the three mappings need distinct workgroup sizes");
// Thresholds (overridable with the environment variables
// MLA_DQ_SMALL_ROWS_MAX, MLA_DQ_MID_ROWS_MAX and MLA_DQ_STREAM_BYTES_MIN,
// read once).
constexpr int64_t kDefaultSmallRowsMax = MLA_DQ_SMALL_ROWS_MAX_DEFAULT;
constexpr int64_t kDefaultSmallRowsMaxFewHeads = MLA_DQ_SMALL_ROWS_MAX_FEW_HEADS_DEFAULT;
constexpr int64_t kFewHeadsMax = MLA_DQ_FEW_HEADS_MAX;
constexpr int64_t kDefaultMidRowsMax = MLA_DQ_MID_ROWS_MAX_DEFAULT;
constexpr int64_t kDefaultStreamBytesMin = MLA_DQ_STREAM_BYTES_MIN_DEFAULT;

constexpr int kMidSizeRowsPerWave = MLA_DQ_MID_SIZE_ROWS_PER_WAVE;
constexpr int64_t kMidSizeBytesMin = MLA_DQ_MID_SIZE_BYTES_MIN;
constexpr int64_t kMidSizeBytesMax = MLA_DQ_MID_SIZE_BYTES_MAX;

constexpr int64_t kRowChunks = 72;   // 576 elements / 8 per 16-byte chunk

struct KernelArgs {
    uint8_t* q_out;
    const uint16_t* ql_nope;
    const uint16_t* q_pe;
    const uint16_t* kv_c;
    const uint16_t* k_pe;
    uint8_t* cache;
    const int64_t* slot_mapping;
    const int64_t* positions;
    const float* rope_cos_sin;
    const float* q_scale;
    const float* kv_scale;
    int64_t ql_nope_st, ql_nope_sh, q_pe_st, q_pe_sh, kv_c_st, k_pe_st;
    int64_t num_slots;
    int64_t max_position;
    FastDiv31 rows_per_token;   // divides a row index by row_stride
    uint32_t num_heads;
    uint32_t total_rows;        // T * row_stride
    uint32_t row_stride;        // rows per token in this launch: H + 1, H (query rows
                                // only) or 1 (cache rows only)
    uint32_t first_head;        // row kind of a token's first row here: 0, or H
                                // (cache rows only); kind H is the cache row
    uint32_t tail_blocks;       // workgroups [0, tail_blocks) do the tails
    uint32_t fp16;              // activations are fp16 (else bf16)
    uint32_t gptj;              // interleaved rotation pairs
    uint32_t table_bf16;        // rope table holds bf16 (else fp32)
};

// The fused product.  Product workgroup g (g < product_blocks, a multiple of
// 8) takes column group g / 8 % column_groups of a unit of XCD g % 8:
// workgroups are dealt to the 8 XCDs round-robin, so the column groups of one
// unit, which read the same q_nope rows, run on one XCD one after another and
// share its L2.  With head_major the unit is (g % 8) * units_per_xcd +
// g / 8 / column_groups, head unit / ranges and token range unit % ranges;
// otherwise it is 8 * (g / 8 / column_groups) + g % 8, head unit % H and
// token range unit / H.  Units past the last exit.
struct UkArgs {
    KernelArgs tails;          // every row's tail (row_stride H + 1)
    KernelArgs cache_rows;     // the cache rows' latent parts (row_stride 1, first_head H)
    const uint16_t* q_nope;
    const uint16_t* w_uk_t;
    int64_t q_nope_st, q_nope_sh;
    FastDiv31 heads;           // divides a unit index by H
    FastDiv31 ranges;          // divides a unit index by the token ranges per head
    uint32_t num_tokens;
    uint32_t tokens_per_group;
    uint32_t units;
    uint32_t units_per_xcd;    // ceil(units / 8)
    uint32_t head_major;       // 1 = head-major unit order (see above)
    uint32_t column_groups;
    uint32_t product_blocks;
    uint32_t tail_blocks;
    uint32_t cache_blocks;
};

constexpr int64_t kDefaultUkLargeRowsMin = MLA_DQ_UK_LARGE_ROWS_MIN_DEFAULT;

// Host-side validation and planning (pure host code, no HIP calls).
int validate(void* q_out, const void* ql_nope, const void* q_pe, const void* kv_c,
             const void* k_pe, void* cache, const int64_t* slot_mapping,
             const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
             const float* kv_scale, uint32_t flags, const mla_dq_dims* dims);
int plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_launch_plan* out);
int64_t row_stride(int64_t H, uint32_t flags);
int uk_validate(void* q_out, const void* q_nope, const void* w_uk_t, const void* q_pe,
                const void* kv_c, const void* k_pe, void* cache, const int64_t* slot_mapping,
                const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
                const float* kv_scale, uint32_t flags, const mla_dq_dims* dims);
int uk_plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_uk_launch_plan* out);

#if defined(__HIPCC__)
hipError_t launch(const KernelArgs& a, const mla_dq_launch_plan& plan, uint32_t flags,
                  hipStream_t stream);
hipError_t launch_uk(const UkArgs& u, const mla_dq_uk_launch_plan& plan, uint32_t flags,
                     hipStream_t stream);
#endif

}  // namespace mla_dq
