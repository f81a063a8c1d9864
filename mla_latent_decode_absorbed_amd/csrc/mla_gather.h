// Internal declarations of the chunked-prefill context kernels: paged gather
// with dequantisation, and the two-way LSE merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct GatherParams {
    const void* kv;             // [num_pages][64][576] bf16 or e4m3
    const float* kv_scale;      // e4m3: device float, the per-tensor cache scale
    const int32_t* block_table; // [batch][max_pages]
    const int32_t* seq_starts;  // [batch]: first gathered token of each request
    const int32_t* cu_lens;     // [batch + 1]: output row offsets (cumulative chunk lengths)
    void* out;                  // [total_rows][576] bf16
    int64_t total_rows;
    int32_t batch, num_pages, max_pages, fp8;
};

struct MergeTwoParams {
    const void* prefix_out;     // [rows][head_dim] fp32 (in_f32) or bf16
    const float* prefix_lse;    // [rows]
    const void* suffix_out;
    const float* suffix_lse;
    void* out;                  // [rows][head_dim] fp32 (out_f32) or bf16
    float* lse;                 // [rows] or null
    int32_t rows, head_dim, in_f32, out_f32;
};

hipError_t launch_gather_cache(const GatherParams& p, hipStream_t stream);
hipError_t launch_merge_two(const MergeTwoParams& p, hipStream_t stream);

}  // namespace mla
