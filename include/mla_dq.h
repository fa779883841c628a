/*
 * mla_dq.h -- C ABI of the fused MLA decode epilogue for AMD MI355X (gfx950).
 *
 * The operation (prhub summary of vLLM PR #54896, "Kimi-K3 MLA decode
 * kernel": sections "implementation breakdown" items 1-3 and "key source
 * snippets"): for every token t, in one launch,
 *
 *   q_out[t, h, 0:512]   = enc_q( ql_nope[t, h, 0:512] )             h < H
 *   q_out[t, h, 512:576] = enc_q( rope(q_pe[t, h, 0:64], pos[t]) )
 *   row(s)[0:512]        = enc_kv( kv_c[t, 0:512] )                  s = slot_mapping[t]
 *   row(s)[512:576]      = enc_kv( rope(k_pe[t, 0:64], pos[t]) )
 *
 * where row(s) is cache[s / block_size, s % block_size, :] of a paged latent
 * cache [num_blocks, block_size, 576].  The page's test fixes the plain case
 * (rotation and FP8 off): q is cat(ql_nope, q_pe) and the cache rows at the
 * slots are cat(kv_c, k_pe); nothing else in the cache changes.
 *
 *   rope(x, p): NeoX half-split rotation; pair k (k < 32) is elements
 *     (k, k+32), or (2k, 2k+1) with MLA_DQ_ROPE_GPTJ, and turns by the angle
 *     whose cos and sin are columns k and 32+k of row p of the caller's
 *     table: first = a*c - b*s, second = b*c + a*s for the pair (a, b), in
 *     fp32, each product and sum rounded separately.  Identity (bit copy)
 *     when MLA_DQ_ROPE is off.
 *   enc (bf16 or fp16 output): bit copy of untouched input, round-to-
 *     nearest-even of rotated fp32 values.
 *   enc (E4M3 output): OCP FP8 E4M3 of fl32(x * fl32(1/scale)) clamped to
 *     [-448, 448] (NaN stays NaN), rounded to nearest even.
 *
 * Conventions where the page is silent:
 *   - slots outside [0, num_blocks*block_size) (e.g. -1 padding) skip the
 *     cache write for that token; the token's q rows are still written;
 *   - positions outside [0, max_position) are clamped into the table;
 *   - valid slots are expected to be unique; with a repeated slot, every
 *     8-element chunk of the row holds that chunk of one of the tokens that
 *     share it, not necessarily the same token for every chunk.
 *
 * Threading and ownership: the library allocates nothing, keeps no state
 * beyond a read-once tuning environment variable, and may be called from
 * several threads.  Every buffer belongs to the caller.  Work is enqueued on
 * `stream` and the call returns without synchronising.
 */
#ifndef MLA_DQ_H
#define MLA_DQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- flags ------------------------------------------------------------- */
/* Feature switches; the page's kernel has the same three as template
 * arguments (section "key source snippets"). */
#define MLA_DQ_ROPE    (1u << 0) /* rotate the 64-wide tails of q and k     */
#define MLA_DQ_Q_FP8   (1u << 1) /* q_out holds E4M3 codes (else bf16)      */
#define MLA_DQ_KV_FP8  (1u << 2) /* cache holds E4M3 codes (else bf16)      */
/* Variants (the page's kernel is templated on the element type; the other
 * two are the common alternatives of the rotary embedding):              */
#define MLA_DQ_FP16       (1u << 3) /* activations, and unquantised q_out and
                                       cache, are fp16 instead of bf16     */
#define MLA_DQ_ROPE_GPTJ  (1u << 4) /* interleaved pairs (2i, 2i+1) instead
                                       of NeoX halves (i, i+32); needs ROPE */
#define MLA_DQ_TABLE_BF16 (1u << 5) /* rope_cos_sin holds bf16 instead of
                                       fp32; needs ROPE                    */
/* Launch overrides for tests and sweeps; they never change the results.
 * By default the library picks, by the row count T * (H + 1), one of three
 * mappings at measured row thresholds: the latency mapping (one latent row
 * per wavefront, 64-thread workgroups) for the fewest rows (up to 896, or
 * up to 2560 with at most 32 heads), the same in 128-thread workgroups
 * next (up to 5120), and the throughput mapping (256-thread
 * workgroups, tails batched, rope table staged in LDS) above; the page's
 * launcher makes the same token-count-dependent choice ("implementation
 * breakdown" items 1 and 3).  Independently, loads and stores stream past
 * the caches (non-temporal) once one call moves at least stream_bytes_min
 * bytes (80 MiB by default, measured inside a decode step; the environment
 * variable MLA_DQ_STREAM_BYTES_MIN overrides it).  At most one mapping
 * override may be set. */
#define MLA_DQ_FORCE_SMALL_T (1u << 8)  /* latency mapping, 64 threads     */
#define MLA_DQ_FORCE_LARGE_T (1u << 9)  /* throughput mapping              */
#define MLA_DQ_FORCE_STREAM  (1u << 10) /* non-temporal loads and stores   */
#define MLA_DQ_FORCE_CACHED  (1u << 11) /* default cache policy            */
#define MLA_DQ_FORCE_MID_T   (1u << 12) /* latency mapping, 128 threads    */
/* Row subsets, for a caller that splits the epilogue around its
 * dependencies.  The cache row of a token needs only kv_c and k_pe, which do
 * not depend on the query projections; the page's kernel lets its cache-row
 * warps skip the wait for the upstream GEMM for that reason
 * ("implementation breakdown" item 2).  With MLA_DQ_Q_ROWS_ONLY the call
 * writes only q_out; with MLA_DQ_CACHE_ROWS_ONLY only the cache rows.  One
 * call of each, in either order or at the same time on two streams, leaves
 * exactly the bytes of one call without them.  The arguments and checks are
 * those of a full call (every pointer the flags require, even those the
 * subset does not read).  At most one of the two. */
#define MLA_DQ_Q_ROWS_ONLY     (1u << 13)
#define MLA_DQ_CACHE_ROWS_ONLY (1u << 14)

/* ---- return codes ------------------------------------------------------ */
#define MLA_DQ_OK          0
#define MLA_DQ_ERR_NULL   -1 /* a required pointer (or dims) is NULL               */
#define MLA_DQ_ERR_ALIGN  -2 /* pointer or stride misaligned (see below)          */
#define MLA_DQ_ERR_DIM    -3 /* a dimension or stride is out of range             */
#define MLA_DQ_ERR_FLAGS  -4 /* unknown flag bit, or contradictory FORCE bits    */
#define MLA_DQ_ERR_LAUNCH -5 /* the HIP launch reported an error                  */
#define MLA_DQ_ERR_ALIAS  -6 /* q_out or the cache overlaps an input that the
                                flags use (activations, slots, positions, rope
                                table, scales), or q_out overlaps the cache    */

/* Shapes and input strides.  Strides are in elements (bf16) and let the
 * inputs be views of larger buffers, as the page's neighbouring GEMM change
 * allows for row-strided activations (prhub summary of vLLM PR #54565,
 * "implementation breakdown" items 1-2): the inner stride is 1 and every row
 * stride is a multiple of 8 elements (16 bytes).  q_out and cache are dense. */
typedef struct mla_dq_dims {
    int64_t num_tokens;       /* T >= 0; T == 0 returns MLA_DQ_OK, no launch   */
    int64_t num_heads;        /* H >= 1                                         */
    int64_t num_blocks;       /* cache blocks, >= 1                             */
    int64_t block_size;       /* slots per block, >= 1                          */
    int64_t max_position;     /* rows of rope_cos_sin; >= 1 when MLA_DQ_ROPE    */
    int64_t ql_nope_stride_t; /* ql_nope[t, h, e] at t*st + h*sh + e            */
    int64_t ql_nope_stride_h;
    int64_t q_pe_stride_t;    /* q_pe[t, h, e] at t*st + h*sh + e               */
    int64_t q_pe_stride_h;
    int64_t kv_c_stride_t;    /* kv_c[t, e] at t*st + e                         */
    int64_t k_pe_stride_t;    /* k_pe[t, e] at t*st + e                         */
} mla_dq_dims;

/*
 * The fused epilogue (prhub summary of vLLM PR #54896: the launcher named in
 * "implementation breakdown" item 3 and the op the test calls in "key source
 * snippets").  All pointers are DEVICE pointers except `dims`, a host pointer.
 *
 *   q_out         [T, H, 576] dense; the activation type (bf16, or fp16 with
 *                 MLA_DQ_FP16), or E4M3 bytes with MLA_DQ_Q_FP8.  16-byte
 *                 aligned.  Written in full.
 *   ql_nope       [T, H, 512] activations (strided, see mla_dq_dims), 16-B
 *                 aligned.
 *   q_pe          [T, H, 64]  activations (strided), 16-B aligned.
 *   kv_c          [T, 512]    activations (strided), 16-B aligned.
 *   k_pe          [T, 64]     activations (strided), 16-B aligned.
 *   cache         [num_blocks, block_size, 576] dense; the activation type,
 *                 or E4M3 bytes with MLA_DQ_KV_FP8.  16-B aligned.  Only the
 *                 rows at valid slots are written.
 *   slot_mapping  int64 [T], 8-B aligned.
 *   positions     int64 [T], 8-B aligned; required with MLA_DQ_ROPE, else
 *                 ignored (may be NULL).
 *   rope_cos_sin  [max_position, 64] fp32 (bf16 with MLA_DQ_TABLE_BF16): row p
 *                 = cos of the 32 angles, then their sin.  16-B aligned;
 *                 required with MLA_DQ_ROPE.
 *   q_scale       fp32 scalar; required with MLA_DQ_Q_FP8 (may be NULL else).
 *   kv_scale      fp32 scalar; required with MLA_DQ_KV_FP8 (may be NULL else).
 *   flags         MLA_DQ_* bits.
 *   dims          host pointer to shapes and strides.
 *   stream        a hipStream_t (NULL = the null stream).
 *
 * Returns MLA_DQ_OK after enqueueing, or a negative MLA_DQ_ERR_* code.  On a
 * validation error nothing is launched; validation reads no device memory.
 */
int mla_decode_q_concat_kv_insert(void* q_out, const void* ql_nope, const void* q_pe,
                                  const void* kv_c, const void* k_pe, void* cache,
                                  const int64_t* slot_mapping, const int64_t* positions,
                                  const float* rope_cos_sin, const float* q_scale,
                                  const float* kv_scale, uint32_t flags,
                                  const mla_dq_dims* dims, void* stream);

/* Human-readable text for a return code; never NULL, static storage. */
const char* mla_dq_strerror(int code);

/* Hexadecimal digest of the source files (kernel sources and these headers)
 * the library was compiled from, fixed at build time; a loader compares it
 * with the sources it ships beside, so that a library built from other
 * sources is refused.  Never NULL, static storage. */
const char* mla_dq_source_digest(void);

/* The launch the library would make for these dims and flags: host-only, no
 * GPU needed, no device memory touched.  The kernel splits every 576-wide
 * row into its 512-wide latent part (64 sixteen-byte chunks: one chunk per
 * lane of one wavefront) and its 64-wide positional tail (8 chunks: 8 lanes,
 * so 8 rows' tails per wavefront). */
typedef struct mla_dq_launch_plan {
    int32_t mapping;          /* 0 = small-T (latency, 64 threads),
                                 1 = large-T (throughput),
                                 2 = mid-T (latency, 128 threads)              */
    int32_t streaming;        /* 1 = non-temporal loads and stores               */
    int32_t block_threads;    /* threads per workgroup (a multiple of 64)        */
    int32_t rows_per_wave;    /* latent rows per wavefront (2 for mid-size calls
                                 of the throughput mapping under the default
                                 cache policy, else 1)                            */
    int32_t tail_steps;       /* steps of 8 tails per wavefront                  */
    int32_t reserved;
    int64_t small_rows_max;   /* row threshold of the small-T mapping in force
                                 for these heads                                  */
    int64_t stream_bytes_min; /* byte threshold in force                         */
    int64_t bytes;            /* bytes the call reads and writes                 */
    int64_t tail_blocks;      /* workgroups doing positional tails (first)       */
    int64_t latent_blocks;    /* workgroups doing latent parts (after them)      */
    int64_t grid_blocks;      /* tail_blocks + latent_blocks                     */
    int64_t total_rows;       /* rows of this launch: T * (H + 1), or T * H with
                                 MLA_DQ_Q_ROWS_ONLY, or T with
                                 MLA_DQ_CACHE_ROWS_ONLY                           */
    int64_t mid_rows_max;     /* row threshold of the mid-T mapping in force     */
} mla_dq_launch_plan;

/* Returns MLA_DQ_OK and fills *plan, or a negative code for bad dims/flags.
 * (Pointers are not checked here; T == 0 gives grid_blocks = 0.) */
int mla_dq_plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_launch_plan* plan);

/* ---- the epilogue fused into the W_UK product ------------------------------
 *
 * In a decode step ql_nope is the output of the per-head absorbed key
 * projection, and the page's kernel starts by waiting for that product
 * ("implementation breakdown" item 2).  This entry point does the product
 * and the epilogue in one launch, so ql_nope is never stored or read back:
 *
 *   ql[t, h, n] = sum over k < 128 of q_nope[t, h, k] * W_UK[h, k, n]     n < 512
 *   q_out[t, h, 0:512] = enc_q( ql[t, h, 0:512] )
 *
 * and everything else (the rotated tails of q, the cache rows) exactly as
 * mla_decode_q_concat_kv_insert writes it.  The sum is formed in fp32 on the
 * matrix cores (bf16 or fp16 products, exact in fp32); its order of
 * additions is the library's, so ql is the exact sum within
 * 2^-16 * sum_k |q_nope[t,h,k] * W_UK[h,k,n]| (well above the fp32 rounding
 * bound of a 128-term sum), and enc_q rounds that fp32 value once: to bf16 /
 * fp16 (nearest even), or to E4M3 of fl32(ql * fl32(1/q_scale)) clamped to
 * [-448, 448].
 *
 *   q_nope   [T, H, 128] activations: element (t, h, k) at
 *            t * dims->ql_nope_stride_t + h * dims->ql_nope_stride_h + k (the
 *            two ql_nope strides of mla_dq_dims describe q_nope here), e.g.
 *            the first 128 of each head's 192 columns of the q projection's
 *            output.  16-B aligned, strides multiples of 8 elements.
 *   w_uk_t   [H, 512, 128] activations, dense: w_uk_t[h, n, k] = W_UK[h, k, n]
 *            (each head's W_UK transposed once, when the weights are loaded,
 *            so that both operands of the product run along k).  16-B aligned.
 *   all other arguments as for mla_decode_q_concat_kv_insert.
 *
 * Flags: MLA_DQ_ROPE, _Q_FP8, _KV_FP8, _FP16 (activations, weights and
 * unquantised outputs fp16), _ROPE_GPTJ, _TABLE_BF16, and the launch
 * overrides MLA_DQ_FORCE_SMALL_T / _FORCE_LARGE_T (latency or throughput
 * configuration, below) and _FORCE_STREAM / _FORCE_CACHED.  The row subsets
 * and MLA_DQ_FORCE_MID_T give MLA_DQ_ERR_FLAGS.  q_out and the cache must not
 * overlap q_nope or w_uk_t either (MLA_DQ_ERR_ALIAS).  Errors and ownership
 * as for mla_decode_q_concat_kv_insert.
 */
int mla_decode_uk_q_concat_kv_insert(void* q_out, const void* q_nope, const void* w_uk_t,
                                     const void* q_pe, const void* kv_c, const void* k_pe,
                                     void* cache, const int64_t* slot_mapping,
                                     const int64_t* positions, const float* rope_cos_sin,
                                     const float* q_scale, const float* kv_scale, uint32_t flags,
                                     const mla_dq_dims* dims, void* stream);

/* The launch of the fused product: host-only, as mla_dq_plan.  One grid of
 * block_threads-thread workgroups holds three kinds: product workgroups
 * first, each for one head, one group of latent columns and a range of
 * tokens (every wavefront holds 16 * n_blocks columns of W_UK in registers
 * and steps through the range 16 tokens at a time, one matrix-core product
 * per 16 x 16 x 32 tile); then the positional tails of all T * (H + 1) rows;
 * then the latent parts of the T cache rows.  The latency configuration
 * (fewest query rows) takes 16 tokens per product workgroup and narrow
 * column groups (n_blocks 2, or 1 when there are at most 32 (head, token
 * range) units), so that even one token spreads over many workgroups; the
 * throughput configuration takes wider groups (n_blocks 4, or 2 with at
 * least 64 tokens and at most 16384 query rows) and longer token ranges (up to 128 tokens, shortened while
 * fewer than about 256 product workgroups would result), so that each q_nope
 * row and each weight row is read fewer times.
 * The throughput configuration is the default from T * H >= large_rows_min
 * (1025, or the environment variable MLA_DQ_UK_LARGE_ROWS_MIN read once);
 * the call streams (non-temporal stores) from stream_bytes_min bytes, the
 * epilogue's threshold (MLA_DQ_STREAM_BYTES_MIN). */
typedef struct mla_dq_uk_launch_plan {
    int32_t mapping;          /* 0 = latency, 1 = throughput                     */
    int32_t streaming;        /* 1 = non-temporal loads and stores               */
    int32_t block_threads;    /* threads per workgroup                           */
    int32_t n_blocks;         /* 16-column blocks of W_UK per wavefront           */
    int32_t tail_steps;       /* steps of 8 tails per wavefront                  */
    int32_t tokens_per_group; /* tokens per product workgroup (a multiple of 16) */
    int64_t column_groups;    /* product workgroups per (head, token range)      */
    int64_t units;            /* H * ceil(T / tokens_per_group)                  */
    int64_t product_blocks;   /* product workgroups (a multiple of 8)            */
    int64_t tail_blocks;      /* workgroups doing positional tails               */
    int64_t cache_blocks;     /* workgroups doing the cache rows' latent parts   */
    int64_t grid_blocks;      /* the sum of the three                            */
    int64_t bytes;            /* bytes the call reads and writes, W_UK once      */
    int64_t flops;            /* 2 * T * H * 128 * 512                           */
    int64_t stream_bytes_min; /* byte threshold in force                         */
    int64_t large_rows_min;   /* T * H from which the throughput configuration
                                 is the default                                  */
    int32_t head_major;       /* 1 = each XCD takes a contiguous block of
                                 (head, token range) units, all ranges of a
                                 head together (from 64 heads); 0 = unit u on
                                 XCD u % 8, ranges outermost                     */
    int32_t reserved;
} mla_dq_uk_launch_plan;

int mla_dq_uk_plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_uk_launch_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DQ_H */
