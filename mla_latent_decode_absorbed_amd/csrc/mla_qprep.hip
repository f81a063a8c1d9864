// gfx950 kernel that prepares the decode query: the per-head absorption of the
// no-rope query part into the latent space, joined with the rope part and
// stored as bf16 or as OCP e4m3 codes under a per-tensor scale.
//
// Decode runs attention in the latent space, so each head's no-rope query
// q_nope[h] (P values) is first mapped through that head's W_UK_T [P][512]
// (a batched matmul over heads: page 1, "实现拆解" item 5; page 4, "MLA
// Prefill vs Decode", the query absorbed into the latent space); the result
// is concatenated with the 64 rope values, as is or quantised to fp8 with a
// per-tensor query scale (page 2, the decode section of the forward_impl
// excerpt, the fused concat + fp8 quantisation of the nope and pe parts).
//
//   q_out[r][h][0:512]   = sum_p q_nope[r][h][p] * W_UK_T[h][p][0:512]
//   q_out[r][h][512:576] = q_pe[r][h][0:64]
//
// Weights are stored latent-major, w_uk[h][l][p] = W_UK_T[h][p][l], so that
// every MFMA operand reads 8 consecutive p values (16 bytes) per lane.
#include "mla_qprep.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

namespace {

typedef __bf16 qp_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 qp_bf16x4 __attribute__((ext_vector_type(4)));
typedef float qp_f32x16 __attribute__((ext_vector_type(16)));
typedef short qp_i16x8 __attribute__((ext_vector_type(8)));

constexpr int kLat = 512;     // latent width
constexpr int kRope = 64;     // rope width
constexpr int kOut = 576;     // prepared row width
constexpr int kChunk = 128;   // latent dims per workgroup (4 waves x 32)
constexpr float kE4m3Max = 448.f;

// fp32 -> OCP e4m3 code, round to nearest even, saturating at +-448 (a
// fixed-scale quantiser clamps to the format's range; gfx950's conversion
// instruction produces OCP e4m3 and rounds to nearest even).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
    b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
    c = fminf(fmaxf(c, -kE4m3Max), kE4m3Max);
    d = fminf(fmaxf(d, -kE4m3Max), kE4m3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Workgroup (head h, latent chunk c) of 4 waves; wave w owns latent dims
// n0 = 128 c + 32 w .. + 31 for every query row.  MFMA v_mfma_f32_32x32x16_bf16
// with the latent dims as M and the query rows as N:
//   D[32 dims][32 rows] += Wt[32 dims][16 p] . Qn^T[16 p][32 rows]
// Lane l supplies row/column l % 32 and k values 8 (l / 32) .. + 7 of both
// operands, and ends with D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i < 16:
// four groups of 4 consecutive latent dims of query row l % 32.
//
// Memory traffic is shaped for HBM and the L2: the workgroup's weight block
// (128 rows x P, contiguous) and each 32-row query tile are loaded with
// consecutive lanes on consecutive 16 bytes (whole 64-byte requests) into LDS
// rows padded by 16 bytes (16 consecutive rows then start on distinct bank
// groups), and the MFMA fragments are read from there; a fragment loaded
// straight from memory would touch 32 rows x 32 bytes per instruction.  The
// loads of the next query tile are issued before the current tile's products.
// Results leave through LDS too: the tile's 32 rows x 128 latent dims are
// stored as whole 256-byte (bf16) or 128-byte (e4m3) row pieces, and each
// row's rope part is written by one workgroup, so HBM sees whole cache lines.
template <int KS>
__global__ __launch_bounds__(256) void query_prep_kernel(QueryPrepParams p) {
    constexpr int P = 16 * KS;
    constexpr int kRowB = 2 * P;            // bytes of one weight or query row
    constexpr int kPad = kRowB + 16;        // LDS row stride
    constexpr int kPieces = kRowB / 16;     // 16-byte pieces per row
    constexpr int kStage = 2 * kChunk + 16; // output staging row stride
    __shared__ __attribute__((aligned(16))) uint8_t w_lds[kChunk * kPad];
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[32 * kPad];
    __shared__ __attribute__((aligned(16))) uint8_t stage[32 * kStage];
    const int h = blockIdx.x >> 2;
    const int chunk = blockIdx.x & 3;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 31;
    const int G = lane >> 5;
    const size_t H = (size_t)p.heads;
    const bool fp8 = p.out_fp8 != 0;

    // rope part: this workgroup writes rows m = chunk + 4 i; thread t takes
    // 16-byte piece t % 8 of row chunk + 4 (t / 8 + 32 j): 8 bf16 values
    auto pe_row = [&](int it) { return chunk + 4 * (it >> 3); };
    const qp_bf16x8* pe_base = (const qp_bf16x8*)((const __bf16*)p.q_pe + (size_t)h * kRope) + (tid & 7);
    qp_bf16x8 pe0;
    if (pe_row(tid) < p.rows) pe0 = pe_base[(size_t)pe_row(tid) * H * (kRope / 8)];

    // the weight block w_uk[h][128 c .. 128 c + 127][0 .. P): contiguous
    constexpr int kWLoads = kChunk * kPieces / 256;   // 16-byte loads per thread
    const uint4* wsrc = (const uint4*)((const uint8_t*)p.w_uk + ((size_t)h * kLat + chunk * kChunk) * kRowB);
    uint4 wreg[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) wreg[j] = wsrc[tid + 256 * j];
    // query tile m0: piece i (< 32 kPieces) is row i / kPieces, piece i % kPieces
    // (rows past the end read the last row; their results are not stored)
    constexpr int kQLoads = (32 * kPieces + 255) / 256;
    struct QTile { uint4 v[kQLoads]; };
    auto load_q = [&](int m0) {
        QTile t;
#pragma unroll
        for (int j = 0; j < kQLoads; ++j) {
            const int i = min(tid + 256 * j, 32 * kPieces - 1);    // (a duplicate load past the tile)
            const int r = i / kPieces, c = i - r * kPieces;
            const int mr = min(m0 + r, p.rows - 1);
            t.v[j] = *((const uint4*)((const uint8_t*)p.q_nope + ((size_t)mr * H + h) * kRowB) + c);
        }
        return t;
    };
    auto put_q = [&](const QTile& t) {
#pragma unroll
        for (int j = 0; j < kQLoads; ++j) {
            const int i = tid + 256 * j;
            if (i < 32 * kPieces) {
                const int r = i / kPieces, c = i - r * kPieces;
                *(uint4*)(q_lds + r * kPad + 16 * c) = t.v[j];
            }
        }
    };
    QTile qreg = load_q(0);
    const float qs = fp8 ? *p.q_scale : 1.f;
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const int i = tid + 256 * j;
        const int r = i / kPieces, c = i - r * kPieces;
        *(uint4*)(w_lds + r * kPad + 16 * c) = wreg[j];
    }
    put_q(qreg);
    __syncthreads();
    // this wave's weight fragments: rows 32 wave + li, p = 16 ks + 8 G ..
    qp_bf16x8 wf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wf[ks] = *(const qp_bf16x8*)(w_lds + (32 * wave + li) * kPad + 32 * ks + 16 * G);
    const int e = fp8 ? 1 : 2;   // bytes per stored value

    for (int m0 = 0; m0 < p.rows; m0 += 32) {
        const bool more = m0 + 32 < p.rows;
        if (more) qreg = load_q(m0 + 32);
        qp_f32x16 acc = (qp_f32x16)0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const qp_bf16x8 qf = *(const qp_bf16x8*)(q_lds + li * kPad + 32 * ks + 16 * G);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], qf, acc, 0, 0, 0);
        }
        // stage: row li, dims 32 wave + 8 g + 4 G .. + 3 of the chunk
        uint8_t* srow = stage + li * kStage + (32 * wave + 4 * G) * e;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float a0 = acc[4 * g], a1 = acc[4 * g + 1], a2 = acc[4 * g + 2], a3 = acc[4 * g + 3];
            if (fp8) {
                *(uint32_t*)(srow + 8 * g) = e4m3_pack4(a0 / qs, a1 / qs, a2 / qs, a3 / qs);
            } else {
                qp_bf16x4 v = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3};
                *(qp_bf16x4*)(srow + 16 * g) = v;
            }
        }
        __syncthreads();   // staged tile complete; every wave is done with q_lds
        // rows m0 .. m0 + 31: 16-byte pieces, 16 (bf16) or 8 (e4m3) per row
        const int per_row = 8 * e;
        for (int i = tid; i < 32 * per_row; i += 256) {
            const int r = i / per_row, c = i - r * per_row;
            const int m = m0 + r;
            if (m < p.rows)
                *(uint4*)((uint8_t*)p.q_out + (((size_t)m * H + h) * kOut + chunk * kChunk) * e + 16 * c) =
                    *(const uint4*)(stage + r * kStage + 16 * c);
        }
        if (more) put_q(qreg);
        __syncthreads();   // the next tile is in q_lds; the staging buffer is free
    }

    auto store_pe = [&](int it, const qp_bf16x8& v) {
        const size_t o = ((size_t)pe_row(it) * H + h) * kOut + kLat + 8 * (it & 7);
        if (fp8) {
            uint2 w;
            w.x = e4m3_pack4((float)v[0] / qs, (float)v[1] / qs, (float)v[2] / qs, (float)v[3] / qs);
            w.y = e4m3_pack4((float)v[4] / qs, (float)v[5] / qs, (float)v[6] / qs, (float)v[7] / qs);
            *(uint2*)((uint8_t*)p.q_out + o) = w;
        } else {
            *(qp_bf16x8*)((__bf16*)p.q_out + o) = v;
        }
    };
    if (pe_row(tid) < p.rows) store_pe(tid, pe0);
    for (int it = tid + 256; pe_row(it) < p.rows; it += 256)
        store_pe(it, pe_base[(size_t)pe_row(it) * H * (kRope / 8)]);
}

}  // namespace

template <int KS>
static void launch_ks(const QueryPrepParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(query_prep_kernel<KS>, dim3((unsigned)(p.heads * 4)), dim3(256), 0, stream, p);
}

hipError_t launch_query_prep(const QueryPrepParams& p, hipStream_t stream) {
    (void)hipGetLastError();   // a stale error of an earlier, unrelated HIP call is not this launch's
    switch (p.nope_dim / 16) {
        case 1: launch_ks<1>(p, stream); break;
        case 2: launch_ks<2>(p, stream); break;
        case 3: launch_ks<3>(p, stream); break;
        case 4: launch_ks<4>(p, stream); break;
        case 5: launch_ks<5>(p, stream); break;
        case 6: launch_ks<6>(p, stream); break;
        case 7: launch_ks<7>(p, stream); break;
        case 8: launch_ks<8>(p, stream); break;
        case 9: launch_ks<9>(p, stream); break;
        case 10: launch_ks<10>(p, stream); break;
        case 11: launch_ks<11>(p, stream); break;
        case 12: launch_ks<12>(p, stream); break;
        case 13: launch_ks<13>(p, stream); break;
        case 14: launch_ks<14>(p, stream); break;
        case 15: launch_ks<15>(p, stream); break;
        case 16: launch_ks<16>(p, stream); break;
        default: return hipErrorInvalidValue;   // the C ABI admits P = 16 .. 256 in steps of 16
    }
    return hipGetLastError();
}

}  // namespace mla
