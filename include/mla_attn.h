/*
 * mla_attn.h -- C ABI of MLA decode attention over the paged latent cache,
 * for AMD MI355X (gfx950).  Same library as mla_dq.h (libmla_dq.so).
 *
 * The consumer of the fused epilogue: the decode step's attention reads the
 * latent query rows q[b, h, 0:576] and the latent cache rows the epilogue
 * wrote (prhub summary of vLLM PR #54896, "implementation breakdown" item 2:
 * the epilogue's output feeds the downstream FMHA).  With absorbed weights
 * every head attends to the same 576-wide cache rows: the key is the whole
 * row, the value its first 512 elements.  For sequence b with L = seq_lens[b]
 * cached tokens:
 *
 *   row_j        = cache[block_table[b, j / block_size], j % block_size, :]
 *   s_j          = sm_scale * sum_d q[b,h,d] * row_j[d]           (d < 576)
 *   out[b,h,:]   = sum_j softmax(s)_j * row_j[0:512]              (0 if L == 0)
 *
 * E4M3 operands count as code * scale (per-tensor scales).  Scores and
 * accumulation are fp32 (bf16 products on matrix cores, probabilities rounded
 * to bf16 for the value product); the output is bf16.
 *
 * The library allocates nothing.  Keys of one sequence are split across
 * workgroups; the partial results live in a caller-provided workspace of
 * mla_decode_attention_workspace_size() bytes.
 */
#ifndef MLA_ATTN_H
#define MLA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ATTN_Q_FP8  (1u << 0) /* q holds E4M3 codes (else bf16)      */
#define MLA_ATTN_KV_FP8 (1u << 1) /* cache holds E4M3 codes (else bf16)  */

/* Return codes are the MLA_DQ_* codes of mla_dq.h (0 success, negative
 * error); mla_dq_strerror() describes them.  -7: workspace too small. */
#define MLA_ATTN_ERR_WORKSPACE -7

typedef struct mla_attn_dims {
    int64_t batch;              /* B >= 0 sequences, one query token each          */
    int64_t num_heads;          /* H >= 1                                          */
    int64_t num_blocks;         /* cache blocks >= 1                               */
    int64_t block_size;         /* tokens per block >= 1                           */
    int64_t max_blocks_per_seq; /* row length of block_table >= 1                  */
    int64_t max_seq_len;        /* every seq_lens[b] <= this, and <= max_blocks_per_seq * block_size */
} mla_attn_dims;

/* Workspace bytes needed for these dims and flags (0 if none is needed, or
 * if dims are invalid).  The split, and so the size, follows the policy read
 * once per process (environment variable MLA_ATTN_TARGET_WGS, else 256
 * workgroups: one per CU). */
size_t mla_decode_attention_workspace_size(const mla_attn_dims* dims, uint32_t flags);

/*
 * out          [B, H, 512] bf16, dense, 16-byte aligned.  Written in full.
 * q            [B, H, 576] bf16 or E4M3 codes (MLA_ATTN_Q_FP8), dense, 16-B aligned.
 * cache        [num_blocks, block_size, 576] bf16 or E4M3 (MLA_ATTN_KV_FP8), dense,
 *              16-B aligned.
 * block_table  int32 [B, max_blocks_per_seq]; entries used for j < seq_lens[b]
 *              must lie in [0, num_blocks) (the kernel clamps them into that range).
 *              Entries past a sequence's length may be read and may hold anything;
 *              neither they nor the cache rows they point to affect the output.
 * seq_lens     int32 [B]; values are clamped into [0, max_seq_len].
 * q_scale, kv_scale: fp32 scalars (device), required with the matching FP8 flag.
 * sm_scale     softmax scale applied to the raw dot products (host value).
 * workspace    device memory of at least mla_decode_attention_workspace_size()
 *              bytes (may be NULL when that size is 0); contents are scratch.
 * All pointers are device pointers except dims (host).  Enqueued on stream;
 * the call returns after the launch, without waiting.  The caller owns every
 * buffer.  out and the workspace must not overlap each other or any input.
 *
 * Returns 0, or (nothing launched; the checks read no device memory):
 *   MLA_DQ_ERR_NULL   (-1) dims NULL, a required pointer NULL (a scale needed
 *                          by its flag, the workspace when one is needed)
 *   MLA_DQ_ERR_ALIGN  (-2) out, q, cache or workspace not 16-byte aligned,
 *                          block_table, seq_lens or a scale not 4-byte aligned
 *   MLA_DQ_ERR_DIM    (-3) a dimension out of range, or sm_scale not finite
 *   MLA_DQ_ERR_FLAGS  (-4) an unknown flag bit
 *   MLA_DQ_ERR_LAUNCH (-5) the HIP launch failed
 *   MLA_DQ_ERR_ALIAS  (-6) out or the workspace overlaps another buffer
 *   MLA_ATTN_ERR_WORKSPACE (-7) workspace_bytes below the size needed
 * batch == 0 returns 0 with no launch.
 */
int mla_decode_attention(void* out, const void* q, const void* cache, const int32_t* block_table,
                         const int32_t* seq_lens, const float* q_scale, const float* kv_scale,
                         float sm_scale, void* workspace, size_t workspace_bytes, uint32_t flags,
                         const mla_attn_dims* dims, void* stream);

/*
 * The same attention for callers that cannot allocate device memory or pass
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, checks and results are those of
 * mla_decode_attention without the workspace.  When the split needs one, the
 * partial results go to a scratch buffer of MLA_ATTN_SCRATCH_BYTES that the
 * library keeps in device memory, one per GPU, from the library's load on
 * that GPU until the process ends.  Nothing is allocated: no hipMalloc,
 * hipFree or allocating library call.
 *
 * MLA_ATTN_SCRATCH_BYTES covers every split of the default plan (at most 510
 * workgroups of 16 heads, 16 776 960 bytes); a plan that needs more (only
 * with MLA_ATTN_TARGET_WGS raised) returns MLA_ATTN_ERR_SCRATCH and launches
 * nothing.  All calls on one GPU share its buffer, which keeps the last
 * call's contents; each call writes every part of it that it reads, so it
 * needs no clearing.  Calls that may overlap on one GPU (on streams without
 * an order between them, or from threads that do not serialise them) race
 * on the buffer: order them.  The buffer used is the one of the GPU that runs
 * stream (the current device for a NULL stream).  Returns the codes of
 * mla_decode_attention except MLA_ATTN_ERR_WORKSPACE, plus:
 *   MLA_ATTN_ERR_SCRATCH (-8) the split needs more than MLA_ATTN_SCRATCH_BYTES
 *   MLA_DQ_ERR_LAUNCH    (-5) also when the buffer's address cannot be found
 */
#define MLA_ATTN_SCRATCH_BYTES (16u << 20)
#define MLA_ATTN_ERR_SCRATCH -8   /* the split needs more than MLA_ATTN_SCRATCH_BYTES */

int mla_decode_attention_noalloc(void* out, const void* q, const void* cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const float* q_scale, const float* kv_scale, float sm_scale,
                                 uint32_t flags, const mla_attn_dims* dims, void* stream);

/* The split of the keys the library would use (host-only, no GPU). */
typedef struct mla_attn_plan {
    int32_t splits;             /* key ranges per sequence                          */
    int32_t keys_per_split;     /* multiple of 64                                   */
    int32_t head_tiles;         /* ceil(H / 16)                                     */
    int32_t combine;            /* 1 = a second pass merges the splits             */
    int64_t workgroups;         /* B * head_tiles * splits                          */
    int64_t workspace_bytes;    /* = mla_decode_attention_workspace_size()         */
    int64_t target_workgroups;  /* policy: 256, or MLA_ATTN_TARGET_WGS if set      */
    int32_t xcd_remap;          /* 1 = head tiles of one key range share an XCD   */
    int32_t block_threads;      /* 256 (bf16 cache, or E4M3 cache with 64-key
                                   ranges: four wavefronts) or 512 (E4M3 cache,
                                   longer ranges: four compute + four loader
                                   wavefronts)                                  */
} mla_attn_plan;

int mla_decode_attention_plan(const mla_attn_dims* dims, uint32_t flags, mla_attn_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ATTN_H */
