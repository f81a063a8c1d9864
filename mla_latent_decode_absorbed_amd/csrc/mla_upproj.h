// Internal declarations of the output up-projection kernel (latent attention
// output through W_UV into the per-head value space).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct UpProjParams {
    const void* o_lat;    // [rows][heads][512] fp32 (in_f32) or bf16
    const void* w_uv;     // [heads][vdim][512] bf16
    void* out;            // [rows][heads][vdim] fp32 (out_f32) or bf16
    int32_t rows, heads, vdim, in_f32, out_f32;
};

hipError_t launch_up_project(const UpProjParams& p, hipStream_t stream);

}  // namespace mla
