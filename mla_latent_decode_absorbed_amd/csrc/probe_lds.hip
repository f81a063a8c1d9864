// LDS read-rate probe: a measurement tool kept out of the decode library
// (built as libmla_probe.so and run by the benchmark's --probe-lds).
//
// One workgroup per CU fills 64 KB of LDS, then every wave reads aligned,
// contiguous blocks (64 lanes x 16 or 8 bytes: no bank conflicts) in an
// unrolled loop with `unroll` reads in flight before the first use, and
// stamps the core clock (s_memtime) around the loop.  The result is the
// median bytes per clock per workgroup, which tells how fast one wave, or
// several waves of one CU, can read LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace {

constexpr int kBlocks = 256;

template <int NT, int U, bool kWide>
__global__ __launch_bounds__(NT) void lds_read_kernel(unsigned long long* clk, uint4* out, int iters) {
    constexpr int kElems = kWide ? 4096 : 8192;        // 64 KB of uint4 or uint2
    __shared__ uint4 buf[4096];
    const int t = threadIdx.x;
    for (int i = t; i < 4096; i += NT) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    uint32_t acc0 = 0, acc1 = 0, acc2 = 0, acc3 = 0;
    const unsigned long long t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            // wave w reads elements 64 w .. 64 w + 63 of a block that moves by
            // 448 elements (a multiple of 64, so blocks stay aligned) per read
            const int e = (t + (it * U + k) * 448) & (kElems - 1);
            if (kWide) {
                const uint4 v = buf[e];
                acc0 ^= v.x; acc1 ^= v.y; acc2 ^= v.z; acc3 ^= v.w;
            } else {
                const uint2 v = reinterpret_cast<const uint2*>(buf)[e];
                acc0 ^= v.x; acc1 ^= v.y;
            }
        }
    }
    __syncthreads();
    const unsigned long long t1 = __builtin_readcyclecounter();
    if (t == 0) clk[blockIdx.x] = t1 - t0;
    out[(size_t)blockIdx.x * NT + t] = make_uint4(acc0, acc1, acc2, acc3);
}

template <int NT, int U, bool kWide>
int run(int iters, double* bytes_per_clk) {
    unsigned long long* clk = nullptr;
    uint4* out = nullptr;
    if (hipMalloc(&clk, kBlocks * sizeof(unsigned long long)) != hipSuccess) return -4;
    if (hipMalloc(&out, (size_t)kBlocks * NT * sizeof(uint4)) != hipSuccess) {
        (void)hipFree(clk);
        return -4;
    }
    int rc = 0;
    for (int rep = 0; rep < 3 && rc == 0; ++rep) {
        hipLaunchKernelGGL((lds_read_kernel<NT, U, kWide>), dim3(kBlocks), dim3(NT), 0, 0, clk, out, iters);
        if (hipDeviceSynchronize() != hipSuccess) rc = -4;
    }
    std::vector<unsigned long long> h(kBlocks);
    if (rc == 0 && hipMemcpy(h.data(), clk, kBlocks * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
        rc = -4;
    (void)hipFree(clk);
    (void)hipFree(out);
    if (rc != 0) return rc;
    std::sort(h.begin(), h.end());
    *bytes_per_clk = (double)iters * U * NT * (kWide ? 16 : 8) / (double)h[kBlocks / 2];
    return 0;
}

}  // namespace

extern "C" {

// Median LDS bytes read per core clock per workgroup (one workgroup per CU,
// 256 workgroups).  threads: 64, 256, 512 or 1024 (waves per CU x 64);
// unroll: 8 or 15 reads in flight; wide: 1 = 16-byte reads, 0 = 8-byte reads.
// Returns 0, -1 for an unsupported combination, -4 for a HIP error.
int mla_probe_lds_read_rate(int threads, int unroll, int wide, double* bytes_per_clk) {
    if (!bytes_per_clk) return -1;
    const int iters = 64000 / (unroll * (threads / 64 > 4 ? threads / 64 : 4));
#define MLA_PROBE_CASE(NT, U)                                                       \
    if (threads == NT && unroll == U)                                               \
        return wide ? run<NT, U, true>(iters, bytes_per_clk) : run<NT, U, false>(iters, bytes_per_clk);
    MLA_PROBE_CASE(64, 8) MLA_PROBE_CASE(64, 15) MLA_PROBE_CASE(256, 8) MLA_PROBE_CASE(256, 15)
    MLA_PROBE_CASE(512, 8) MLA_PROBE_CASE(512, 15) MLA_PROBE_CASE(1024, 8) MLA_PROBE_CASE(1024, 15)
#undef MLA_PROBE_CASE
    return -1;
}

}  // extern "C"
