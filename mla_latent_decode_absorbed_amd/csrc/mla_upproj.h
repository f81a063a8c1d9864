// Internal declarations of the output up-projection kernel (latent attention
// output through W_UV into the per-head value space).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Upper bound on the partials one fused merge + up-projection takes.
constexpr int kMaxMergeUp = 16;

struct UpProjParams {
    const void* o_lat;    // [rows][heads][512] fp32 (in_f32) or bf16; with n_merge > 0:
                          // n_merge stacked fp32 partials [n][rows * heads][512]
    const float* lses;    // n_merge > 0: [n][rows * heads] natural-log LSEs of the partials
    float* lse_out;       // n_merge > 0: merged LSE [rows * heads], or null
    const void* w_uv;     // [heads][vdim][512] bf16
    void* out;            // [rows][heads][vdim] fp32 (out_f32) or bf16
    int32_t rows, heads, vdim, in_f32, out_f32, n_merge;
};

hipError_t launch_up_project(const UpProjParams& p, hipStream_t stream);

}  // namespace mla
