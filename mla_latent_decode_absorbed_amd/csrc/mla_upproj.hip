// gfx950 kernel for the output up-projection: each head's 512-dim latent
// attention output is mapped through that head's W_UV into its v_head_dim
// value space, the attention layer's output shape (page 1, "关键源码片段",
// output_shape = tokens x num_heads * v_head_dim; page 4, "MLA Prefill vs
// Decode": W_UV decompresses the latent into per-head values).
//
//   out[r][h][v] = sum_l W_UV[h][v][l] * o_lat[r][h][l]
//
// The latent output arrives in fp32 (the decode's and the merge's default) or
// bf16.  A bf16 MFMA takes an fp32 input as two bf16 terms, hi = bf16(x) and
// lo = bf16(x - hi), which carry x to within 2^-17 of its magnitude; both
// terms go through the same weights, so the sum keeps near-fp32 accuracy at
// twice the (here negligible) matrix work.
#include "mla_upproj.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mla {

namespace {

typedef __bf16 up_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 up_bf16x4 __attribute__((ext_vector_type(4)));
typedef float up_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLat = 512;       // latent width (the contraction)
constexpr int kKc = 128;        // latent dims per K chunk
constexpr int kVc = 128;        // value dims per workgroup (4 waves x 32)
constexpr int kPad = 2 * kKc + 16;   // LDS row stride of a bf16 K-chunk row (272 B)

// Workgroup (head h, value chunk vc, row tile mt) of 4 waves; wave w owns
// value dims v0 = 128 vc + 32 w .. + 31.  MFMA v_mfma_f32_32x32x16_bf16 with
// the value dims as M and the rows as N:
//   D[32 v][32 rows] += W_UV[h][32 v][16 l] . O^T[16 l][32 rows]
// Lane l supplies row/column l % 32 and k values 8 (l / 32) .. + 7 of both
// operands, and ends with D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i < 16.
// The weight block (128 v x 512 l) and the row tile (32 rows) pass through
// LDS one K chunk of 128 latent dims at a time, loaded with consecutive lanes
// on consecutive 16 bytes, in rows padded by 16 bytes (16 consecutive rows
// start on distinct bank groups).  Workgroups that share a weight block (same h, vc; other
// row tiles) run on one XCD, so the block comes from that XCD's L2.
// MODE 0: bf16 latent input; 1: fp32 latent input; 2: the latent input is the
// LSE merge of n_merge fp32 partials (mla_merge_states fused in front: each
// row's weights exp(lse_i - max) / sum come first, then every K chunk of the
// row tile is the weighted sum of the partials' chunks, so the merged latent
// never goes through HBM).
template <int MODE>
__global__ __launch_bounds__(256) void up_project_kernel(UpProjParams p) {
    constexpr bool IN_F32 = MODE != 0;
    __shared__ __attribute__((aligned(16))) uint8_t w_lds[kVc * kPad];
    __shared__ __attribute__((aligned(16))) uint8_t hi_lds[32 * kPad];
    __shared__ __attribute__((aligned(16))) uint8_t lo_lds[IN_F32 ? 32 * kPad : 16];
    constexpr int kStage = 4 * kVc + 16;                 // fp32 output row stride
    __shared__ __attribute__((aligned(16))) uint8_t stage[32 * kStage];

    const int vchunks = (p.vdim + kVc - 1) / kVc;
    const int mtiles = (p.rows + 31) / 32;
    const int u = blockIdx.x;
    const int x = u & 7, q = u >> 3;
    const int mt = q % mtiles;
    const int hv = (q / mtiles) * 8 + x;
    if (hv >= p.heads * vchunks) return;                 // (whole workgroup: no barrier is skipped by part of it)
    const int h = hv / vchunks, vc = hv - h * vchunks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, G = lane >> 5;
    const int m0 = 32 * mt;
    const int vrows = min(kVc, p.vdim - kVc * vc);       // valid value rows of this chunk (multiple of 32)
    const bool wave_on = 32 * wave < vrows;
    const size_t H = (size_t)p.heads;

    // merge weights of the tile's rows (MODE 2): row li's weight of partial i
    // at mw[li][i]; a row whose partials are all empty gets weights 0 (out 0,
    // LSE -inf)
    __shared__ float mw[MODE == 2 ? 32 : 1][MODE == 2 ? kMaxMergeUp : 1];
    const size_t rows_all = (size_t)p.rows * H;
    if (MODE == 2) {
        if (tid < 32) {
            const int m = min(m0 + tid, p.rows - 1);
            const size_t row = (size_t)m * H + h;
            float mx = -INFINITY;
            for (int i = 0; i < p.n_merge; ++i) mx = fmaxf(mx, p.lses[i * rows_all + row]);
            float sum = 0.f;
            for (int i = 0; i < p.n_merge; ++i) {
                const float li = p.lses[i * rows_all + row];
                const float wgt = (mx == -INFINITY || li == -INFINITY) ? 0.f : expf(li - mx);
                mw[tid][i] = wgt;
                sum += wgt;
            }
            const float inv = sum > 0.f ? 1.f / sum : 0.f;
            for (int i = 0; i < p.n_merge; ++i) mw[tid][i] *= inv;
            if (p.lse_out && vc == 0 && m0 + tid < p.rows)
                p.lse_out[row] = mx == -INFINITY ? -INFINITY : mx + logf(sum);
        }
        __syncthreads();
    }

    // K chunk kc: weight piece i = tid + 256 j is (v row i / 16, 16 B piece
    // i % 16); row-tile piece i is fp32 (row i / 32, 4 floats i % 32) or bf16
    // (row i / 16, 8 values i % 16).  Each chunk's loads live in registers only
    // until they are written to LDS; the two workgroups a CU holds overlap
    // each other's memory round trips.
    constexpr int kChunks = kLat / kKc;
    constexpr int kOLoads = IN_F32 ? 4 : 2;
    constexpr int kEl = IN_F32 ? 4 : 2;
    up_f32x16 acc = (up_f32x16)0.f;
#pragma unroll
    for (int kc = 0; kc < kChunks; ++kc) {
        uint4 wv[8];
        uint4 ov[kOLoads];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = tid + 256 * j;
            const int r = min(i >> 4, vrows - 1), pc = i & 15;
            wv[j] = *((const uint4*)((const __bf16*)p.w_uv + ((size_t)h * p.vdim + kVc * vc + r) * kLat + kKc * kc) + pc);
        }
        if (MODE != 2) {
#pragma unroll
            for (int j = 0; j < kOLoads; ++j) {
                const int i = tid + 256 * j;
                const int r = IN_F32 ? i >> 5 : i >> 4, pc = IN_F32 ? i & 31 : i & 15;
                const int mr = min(m0 + r, p.rows - 1);
                const uint8_t* row = (const uint8_t*)p.o_lat + ((size_t)mr * H + h) * kLat * kEl;
                ov[j] = *((const uint4*)(row + kKc * kc * kEl) + pc);
            }
        } else {
            // weighted sum of the partials' pieces, four partials' loads in
            // flight at a time; a zero weight (an empty partial) is never read
            float4 acc4[kOLoads];
#pragma unroll
            for (int j = 0; j < kOLoads; ++j) acc4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int i0 = 0; i0 < p.n_merge; i0 += 4) {
                uint4 pv[4][kOLoads];
                float wv[4][kOLoads];
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < kOLoads; ++j) {
                        const int i = tid + 256 * j;
                        const int r = i >> 5, pc = i & 31;
                        const int mr = min(m0 + r, p.rows - 1);
                        wv[k][j] = i0 + k < p.n_merge ? mw[r][i0 + k] : 0.f;
                        const float* row = (const float*)p.o_lat + ((size_t)(i0 + k) * rows_all + (size_t)mr * H + h) * kLat;
                        pv[k][j] = wv[k][j] != 0.f ? *((const uint4*)(row + kKc * kc) + pc) : make_uint4(0, 0, 0, 0);
                    }
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < kOLoads; ++j) {
                        const float wgt = wv[k][j];
                        acc4[j].x += wgt * __uint_as_float(pv[k][j].x);
                        acc4[j].y += wgt * __uint_as_float(pv[k][j].y);
                        acc4[j].z += wgt * __uint_as_float(pv[k][j].z);
                        acc4[j].w += wgt * __uint_as_float(pv[k][j].w);
                    }
            }
#pragma unroll
            for (int j = 0; j < kOLoads; ++j)
                ov[j] = make_uint4(__float_as_uint(acc4[j].x), __float_as_uint(acc4[j].y),
                                   __float_as_uint(acc4[j].z), __float_as_uint(acc4[j].w));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = tid + 256 * j;
            *(uint4*)(w_lds + (i >> 4) * kPad + 16 * (i & 15)) = wv[j];
        }
#pragma unroll
        for (int j = 0; j < kOLoads; ++j) {
            const int i = tid + 256 * j;
            if (IN_F32) {
                const int r = i >> 5, pc = i & 31;
                const float f0 = __uint_as_float(ov[j].x), f1 = __uint_as_float(ov[j].y);
                const float f2 = __uint_as_float(ov[j].z), f3 = __uint_as_float(ov[j].w);
                const __bf16 h0 = (__bf16)f0, h1 = (__bf16)f1, h2 = (__bf16)f2, h3 = (__bf16)f3;  // nearest even
                const up_bf16x4 hv4 = {h0, h1, h2, h3};
                // the differences are exact in fp32; their bf16 rounding is the lo term
                const up_bf16x4 lv4 = {(__bf16)(f0 - (float)h0), (__bf16)(f1 - (float)h1),
                                       (__bf16)(f2 - (float)h2), (__bf16)(f3 - (float)h3)};
                *(up_bf16x4*)(hi_lds + r * kPad + 8 * pc) = hv4;
                *(up_bf16x4*)(lo_lds + r * kPad + 8 * pc) = lv4;
            } else {
                *(uint4*)(hi_lds + (i >> 4) * kPad + 16 * (i & 15)) = ov[j];
            }
        }
        __syncthreads();
        if (wave_on) {
#pragma unroll
            for (int ks = 0; ks < kKc / 16; ++ks) {
                const up_bf16x8 a = *(const up_bf16x8*)(w_lds + (32 * wave + li) * kPad + 32 * ks + 16 * G);
                const up_bf16x8 bh = *(const up_bf16x8*)(hi_lds + li * kPad + 32 * ks + 16 * G);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
                if (IN_F32) {
                    const up_bf16x8 bl = *(const up_bf16x8*)(lo_lds + li * kPad + 32 * ks + 16 * G);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // stage the tile (row li, value dims 32 wave + 8 g + 4 G .. + 3) as fp32,
    // then store whole row pieces in the output type
    if (wave_on) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(float4*)(stage + li * kStage + 4 * (32 * wave + 8 * g + 4 * G)) =
                make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    }
    __syncthreads();
    const int per_row = vrows / 4;                       // 16-byte fp32 pieces per row
    for (int i = tid; i < 32 * per_row; i += 256) {
        const int r = i / per_row, c = i - r * per_row;
        const int m = m0 + r;
        if (m >= p.rows) continue;
        const float4 v = *(const float4*)(stage + r * kStage + 16 * c);
        const size_t o = ((size_t)m * H + h) * p.vdim + kVc * vc + 4 * c;
        if (p.out_f32) {
            *(float4*)((float*)p.out + o) = v;
        } else {
            up_bf16x4 b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
            *(up_bf16x4*)((__bf16*)p.out + o) = b;
        }
    }
}

}  // namespace

hipError_t launch_up_project(const UpProjParams& p, hipStream_t stream) {
    const int vchunks = (p.vdim + kVc - 1) / kVc;
    const int mtiles = (p.rows + 31) / 32;
    const int groups = (p.heads * vchunks + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * mtiles));
    (void)hipGetLastError();   // a stale error of an earlier, unrelated HIP call is not this launch's
    if (p.n_merge > 0) hipLaunchKernelGGL(up_project_kernel<2>, grid, dim3(256), 0, stream, p);
    else if (p.in_f32) hipLaunchKernelGGL(up_project_kernel<1>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(up_project_kernel<0>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
