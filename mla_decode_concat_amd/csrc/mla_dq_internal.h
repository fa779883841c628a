// Internal declarations shared by the launch code and the kernel file.
#pragma once

#include <stdint.h>

#include "mla_dq.h"
#include "fastdiv.h"

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#endif

namespace mla_dq {

// Mapping parameters: chunks (16-byte bf16 loads) per lane and threads per
// workgroup, for the latency mapping and the throughput mapping.
constexpr int kSmallCpl = 1;
constexpr int kSmallBlock = 64;
constexpr int kLargeCpl = 4;
constexpr int kLargeBlock = 256;
// Default token threshold between the two (overridable with the
// environment variable MLA_DQ_SMALL_T_MAX, read once).
constexpr int kDefaultSmallTMax = 64;

constexpr int64_t kRowChunks = 72;   // 576 elements / 8 per chunk

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
    FastDiv31 rows_per_token;   // divides a row index by H + 1
    uint32_t num_heads;
    uint32_t total_chunks;
};

// Host-side validation and planning (pure host code, no HIP calls).
int validate(void* q_out, const void* ql_nope, const void* q_pe, const void* kv_c,
             const void* k_pe, void* cache, const int64_t* slot_mapping,
             const int64_t* positions, const float* rope_cos_sin, const float* q_scale,
             const float* kv_scale, uint32_t flags, const mla_dq_dims* dims);
int plan(const mla_dq_dims* dims, uint32_t flags, mla_dq_launch_plan* out);

#if defined(__HIPCC__)
hipError_t launch(const KernelArgs& a, const mla_dq_launch_plan& plan, uint32_t flags,
                  hipStream_t stream);
#endif

}  // namespace mla_dq
