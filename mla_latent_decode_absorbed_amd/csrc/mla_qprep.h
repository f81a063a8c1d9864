// Internal declarations of the query-preparation kernel (absorption of the
// no-rope query through W_UK_T, rope concatenation, bf16 / e4m3 storage).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct QueryPrepParams {
    const void* q_nope;   // [rows][heads][nope_dim] bf16
    const void* q_pe;     // [rows][heads][64] bf16
    const void* w_uk;     // [heads][512][nope_dim] bf16, w_uk[h][l][p] = W_UK_T[h][p][l]
    const float* q_scale; // fp8 output: device float, the per-tensor query scale
    void* q_out;          // [rows][heads][576] bf16 or e4m3
    int32_t rows, heads, nope_dim, out_fp8;
};

hipError_t launch_query_prep(const QueryPrepParams& p, hipStream_t stream);

}  // namespace mla
