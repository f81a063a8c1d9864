// gfx950 kernels for the chunked-prefill context path that shares the paged
// latent cache and the LSE merge with decode:
//
//   gather_cache_kernel - the latent rows of each request's context chunk
//       (tokens seq_starts[b] .. + len_b - 1) out of the paged cache into one
//       contiguous bf16 buffer, dequantising an e4m3 cache with its
//       per-tensor scale (page 4, "与非 DCP 的流程对比":
//       gather_and_maybe_dequant_cache; page 2, "实现拆解" items 3 and 4: the
//       gather whose requests start at seq_starts);
//   merge_two_kernel - merge_attn_states of a prefix and a suffix partial
//       result (page 4, "Chunked Prefill 与 LSE Merge").
#include "mla_gather.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mla {

namespace {

typedef __bf16 g_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 g_bf16x4 __attribute__((ext_vector_type(4)));
typedef float g_f32x2 __attribute__((ext_vector_type(2)));

constexpr int kQKg = 576;                 // values per cache row
constexpr int kPageTok = 64;              // tokens per page
constexpr int kPieces = kQKg / 8;         // 16-byte bf16 output pieces per row (72)
// Rows per workgroup: 128 for a bf16 cache, 64 for e4m3 (measured best of
// 16 / 32 / 64 / 128 for each; 16 was 6-8 % slower for both).
constexpr int kRowsPerWgBf16 = 128;
constexpr int kRowsPerWgFp8 = 64;

// Workgroup g writes output rows R g .. R g + R - 1 (R = kRowsPerWg).  Threads
// 0..R-1 first find their row's source (request by binary search over the
// cumulative chunk lengths, then token, page id and row in page) and publish
// it in LDS; then every thread copies 16-byte pieces (bf16) or dequantises 16
// codes into 32 bytes (e4m3), consecutive threads on consecutive pieces of a
// row.  A row whose token lies past the block table, or whose page id is
// outside the pool, is written as zeros (a bad table entry never turns into a
// wild read).
template <int kRowsPerWg>
__global__ __launch_bounds__(256) void gather_cache_kernel(GatherParams p) {
    static_assert(kRowsPerWg <= 256, "one source lookup per thread");
    __shared__ const uint8_t* src_row[kRowsPerWg];
    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWg;
    const int e = p.fp8 ? 1 : 2;
    if (tid < kRowsPerWg) {
        const int64_t r = row0 + tid;
        const uint8_t* src = nullptr;
        if (r < p.total_rows) {
            // largest b with cu[b] <= r (cu is non-decreasing, cu[0] = 0)
            int lo = 0, hi = p.batch;                    // invariant: cu[lo] <= r, answer in [lo, hi)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)p.cu_lens[mid] <= r) lo = mid; else hi = mid;
            }
            const int b = lo;
            if (r < (int64_t)p.cu_lens[b + 1]) {
                const int64_t t = (int64_t)p.seq_starts[b] + (r - p.cu_lens[b]);
                const int64_t pg = t / kPageTok;
                if (t >= 0 && pg < p.max_pages) {
                    const int pid = p.block_table[(size_t)b * p.max_pages + pg];
                    if (pid >= 0 && pid < p.num_pages)
                        src = (const uint8_t*)p.kv + ((size_t)pid * kPageTok + (t % kPageTok)) * kQKg * e;
                }
            }
        }
        src_row[tid] = src;
    }
    __syncthreads();
    if (p.fp8) {
        // 16 e4m3 codes per thread and step (a 16-byte load, two 16-byte
        // stores): code -> fp32 (exact) -> * scale (fp32) -> bf16, nearest even
        const float scale = *p.kv_scale;
        constexpr int kJobs = kQKg / 16;              // 36 per row
        for (int i = tid; i < kRowsPerWg * kJobs; i += 256) {
            const int rr = i / kJobs, c = i - rr * kJobs;
            const int64_t r = row0 + rr;
            if (r >= p.total_rows) break;
            const uint8_t* src = src_row[rr];
            uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
            if (src) {
                const uint4 w = *(const uint4*)(src + 16 * c);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                g_bf16x8 o[2];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const g_f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[k], false);
                    const g_f32x2 b2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[k], true);
                    o[k >> 1][4 * (k & 1) + 0] = (__bf16)(a.x * scale);
                    o[k >> 1][4 * (k & 1) + 1] = (__bf16)(a.y * scale);
                    o[k >> 1][4 * (k & 1) + 2] = (__bf16)(b2.x * scale);
                    o[k >> 1][4 * (k & 1) + 3] = (__bf16)(b2.y * scale);
                }
                lo = __builtin_bit_cast(uint4, o[0]);
                hi = __builtin_bit_cast(uint4, o[1]);
            }
            uint4* dst = (uint4*)((uint8_t*)p.out + ((size_t)r * kQKg) * 2 + 32 * c);
            dst[0] = lo;
            dst[1] = hi;
        }
        return;
    }
    for (int i = tid; i < kRowsPerWg * kPieces; i += 256) {
        const int rr = i / kPieces, c = i - rr * kPieces;
        const int64_t r = row0 + rr;
        if (r >= p.total_rows) break;
        const uint8_t* src = src_row[rr];
        const uint4 v = src ? *(const uint4*)(src + 16 * c) : make_uint4(0, 0, 0, 0);
        *(uint4*)((uint8_t*)p.out + ((size_t)r * kQKg) * 2 + 16 * c) = v;
    }
}

// One thread per 4 consecutive elements of a row: both LSEs of its row, the
// weights exp(lse_i - max), and out = (w_p prefix + w_s suffix) / (w_p + w_s);
// the thread holding a row's first element writes lse = max + ln(w_p + w_s).
// A -inf LSE marks an empty partial (weight 0; its output is never read); two
// empty inputs give out = 0 and lse = -inf.
__global__ __launch_bounds__(256) void merge_two_kernel(MergeTwoParams p) {
    const int quads = p.head_dim / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.rows * quads) return;
    const int64_t row = idx / quads;
    const int q = (int)(idx - row * quads);
    const float lp = p.prefix_lse[row], ls = p.suffix_lse[row];
    const float mx = fmaxf(lp, ls);
    const size_t off = (size_t)row * p.head_dim + 4 * q;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float sum = 0.f;
    if (mx != -INFINITY) {
        const float wp = lp == -INFINITY ? 0.f : expf(lp - mx);
        const float ws = ls == -INFINITY ? 0.f : expf(ls - mx);
        sum = wp + ws;
        auto load4 = [&](const void* base) -> float4 {
            if (p.in_f32) return *(const float4*)((const float*)base + off);
            const g_bf16x4 v = *(const g_bf16x4*)((const __bf16*)base + off);
            return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
        };
        const float inv = 1.f / sum;
        if (wp != 0.f) {
            const float4 a = load4(p.prefix_out);
            const float f = wp * inv;
            o.x += f * a.x; o.y += f * a.y; o.z += f * a.z; o.w += f * a.w;
        }
        if (ws != 0.f) {
            const float4 a = load4(p.suffix_out);
            const float f = ws * inv;
            o.x += f * a.x; o.y += f * a.y; o.z += f * a.z; o.w += f * a.w;
        }
    }
    if (p.out_f32) {
        *(float4*)((float*)p.out + off) = o;
    } else {
        const g_bf16x4 b = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
        *(g_bf16x4*)((__bf16*)p.out + off) = b;
    }
    if (p.lse && q == 0) p.lse[row] = mx == -INFINITY ? -INFINITY : mx + logf(sum);
}

}  // namespace

// Each launcher reads hipGetLastError() once before its launch, so that a
// stale error left by an unrelated earlier HIP call is not reported as this
// launch's failure, and once after it for the launch's own status.
hipError_t launch_gather_cache(const GatherParams& p, hipStream_t stream) {
    (void)hipGetLastError();
    if (p.fp8) {
        const int64_t groups = (p.total_rows + kRowsPerWgFp8 - 1) / kRowsPerWgFp8;
        hipLaunchKernelGGL(gather_cache_kernel<kRowsPerWgFp8>, dim3((unsigned)groups), dim3(256), 0, stream, p);
    } else {
        const int64_t groups = (p.total_rows + kRowsPerWgBf16 - 1) / kRowsPerWgBf16;
        hipLaunchKernelGGL(gather_cache_kernel<kRowsPerWgBf16>, dim3((unsigned)groups), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_merge_two(const MergeTwoParams& p, hipStream_t stream) {
    const int64_t threads = (int64_t)p.rows * (p.head_dim / 4);
    (void)hipGetLastError();
    hipLaunchKernelGGL(merge_two_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
