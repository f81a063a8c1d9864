// gfx950 (CDNA4) kernels for absorbed-MQA MLA decode over a paged latent cache.
//
// The cache is ONE latent head of 576 values per token, the query is already
// absorbed into the same 576-dim space, and V is the first 512 dims of the same
// rows (page 4, "MLA Prefill vs Decode").  Every (request, query token, head)
// row attends to the request's cache tokens; heads x query tokens form the M
// dimension of two dense contractions per 64-token page:
//     S^T[token][row] = K[token][0:576] . Q[row][0:576]       (MFMA, K from LDS)
//     O^T[dim][row]  += V^T[dim][token] . P^T[token][row]     (MFMA, V via LDS transpose reads)
// with an online softmax in between.  The call returns output AND log-sum-exp
// (page 2, forward_mqa), split-KV partials are merged by LSE rescaling (page 4,
// "Chunked Prefill 与 LSE Merge"), and the same merge combines DCP shards
// (page 4, "DCP 在 Prefill 与 Decode 中的不同角色").
//
// Kernels:
//   plan_kernel     - reads seq_lens on the device, chooses splits, writes the work list
//   decode_bf16     - one workgroup per work item: streams pages HBM -> LDS, QK^T, softmax, PV
//   combine_kernel  - LSE-merges the split partials of each row into the shard result
//   merge_kernel    - LSE-merges n stacked partial results (DCP shards)

#include "mla_internal.h"

#include <math.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = kQK * 2;                 // 1152 bytes per bf16 cache row
constexpr int kPageBytes = kPage * kRowBytes;      // 73728 bytes per bf16 page
constexpr int kRowChunks = kRowBytes / 16;         // 72 16-byte chunks per row
constexpr int kPageChunks = kPage * kRowChunks;    // 4608 chunks per page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// LDS page layout: row t (token) of 1152 bytes, its 16-byte chunks permuted
// within aligned groups of 8 by c -> c ^ swz(t).  swz maps 8 consecutive tokens
// to 8 distinct values (row-fragment reads of 8 tokens x 16 B hit distinct
// banks) and 4 consecutive tokens to 4 distinct even values (transpose reads of
// 4 tokens x 2 chunks hit distinct banks).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ int lds_off(int t, int c) { return t * kRowBytes + ((c ^ swz(t)) << 4); }

// ---------------------------------------------------------------------------
// plan: per-request split counts and the work list (one workgroup, no host sync)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p, const int32_t* __restrict__ seq_lens,
                                                    int32_t* __restrict__ req_info,
                                                    WorkItem* __restrict__ work) {
    __shared__ long long s_red[1024];
    __shared__ int s_scan[1024];
    const int tid = threadIdx.x;
    const int per = (p.batch + 1023) / 1024;
    const int b0 = min(p.batch, tid * per), b1 = min(p.batch, b0 + per);
    const int cap = p.max_pages * kPage;

    long long my_pages = 0;
    for (int b = b0; b < b1; ++b) {
        int n = min(max(seq_lens[b], 0), cap);
        my_pages += (n + kPage - 1) / kPage;
    }
    s_red[tid] = my_pages;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (tid < s) s_red[tid] += s_red[tid + s];
        __syncthreads();
    }
    const long long total_pages = s_red[0];
    long long chunk = 1;
    if (p.num_splits <= 0) {
        long long want = (total_pages * p.m_tiles + p.target_units - 1) / p.target_units;
        chunk = want > p.min_chunk ? want : p.min_chunk;
    }

    int my_k = 0;
    for (int b = b0; b < b1; ++b) {
        int n = min(max(seq_lens[b], 0), cap);
        int pages = (n + kPage - 1) / kPage;
        int S = p.num_splits > 0 ? min(p.num_splits, pages) : (int)((pages + chunk - 1) / chunk);
        my_k += max(S, 1);
    }
    s_scan[tid] = my_k;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
        int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const int k_total = s_scan[1023];
    int base = s_scan[tid] - my_k;

    for (int b = b0; b < b1; ++b) {
        int n = min(max(seq_lens[b], 0), cap);
        int pages = (n + kPage - 1) / kPage;
        int S, cb;
        if (p.num_splits > 0) {
            S = max(1, min(p.num_splits, pages));
            cb = (pages + S - 1) / S;
        } else {
            S = max(1, (int)((pages + chunk - 1) / chunk));
            cb = (int)chunk;
        }
        req_info[2 * b] = S;
        req_info[2 * b + 1] = base;
        for (int s = 0; s < S; ++s) {
            const int k = base + s;
            const int pb = min(pages, s * cb), pe = min(pages, (s + 1) * cb);
            for (int mt = 0; mt < p.m_tiles; ++mt) {
                WorkItem w;
                w.b = b; w.mt = mt; w.split = s; w.page_begin = pb; w.page_end = pe;
                w.nsplit = S; w.pad0 = 0; w.pad1 = 0;
                work[unit_index(k, mt, p.m_tiles)] = w;
            }
        }
        base += S;
    }
    // slots past the last kv-unit are empty
    for (int u = tid; u < p.units_max; u += 1024) {
        const int grp = u / (8 * p.m_tiles);
        const int k = grp * 8 + (u & 7);
        if (k >= k_total) {
            WorkItem w;
            w.b = -1; w.mt = 0; w.split = 0; w.page_begin = 0; w.page_end = 0;
            w.nsplit = 0; w.pad0 = 0; w.pad1 = 0;
            work[u] = w;
        }
    }
}

// ---------------------------------------------------------------------------
// split-KV decode, bf16 cache
//
// Workgroup = 4 waves (one per SIMD) = 2 pairs; a pair owns 32 query rows, so
// kMTile = 64.  One work item (request, M-tile, page range) per workgroup.
// Both contractions use v_mfma_f32_32x32x16_bf16 with the query rows as the
// MFMA N dimension, so every K or V fragment read from LDS feeds 32 rows:
//   S^T[32 tok][32 rows]  += K[32 tok][16 dims]  . Q^T[16 dims][32 rows]
//   O^T[32 dims][32 rows] += V^T[32 dims][16 tok] . P^T[16 tok][32 rows]
// The cache streams through LDS in half pages of 32 tokens (36,864 bytes)
// held in a ring of 4 slots: three half pages are in flight while one is used.
// Within a pair, wave h contracts dims 288h .. 288h+287 of every token of the
// half page; the pair adds its two partial S^T tiles through LDS (IEEE
// addition is commutative, so both waves hold bit-identical S), both run the
// same online softmax, and wave h accumulates O^T for dims 256h .. 256h+255.
// Each lane owns one query row (lane % 32).  The wave's Q^T half (72 VGPRs)
// and O^T half (128 accumulators) stay in registers for the whole range.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kHalfTok = 32;                          // tokens per ring slot
constexpr int kSlotBytes = kHalfTok * kRowBytes;      // 36,864
constexpr int kSlots = 4;
constexpr int kDmaPerHalf = 9;                        // 1 KB direct loads per wave per half page
constexpr float kRescaleSlack = 8.f;                  // lazy max: rescale when the max grows by > 2^8

// One direct HBM -> LDS load of 16 bytes per lane: lane i writes LDS bytes
// [lds_addr + 16 i, +16) with the 16 bytes at gbase + voff.  Issued as inline
// assembly so that the compiler does not track it: the caller waits for it
// explicitly before the data is read, and the compiler's own LDS waits stay
// exact instead of draining every pending LDS read.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* gbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// Copy one half page (32 tokens) into a ring slot.  LDS chunk q = 64 j + lane
// of instruction j of 8-token group g holds (token q / 72, position q % 72) =
// global chunk (position ^ swz(token)) of that token; wave w copies group w.
__device__ __forceinline__ void issue_half_copy(uint32_t slot_addr, const uint8_t* half_src, int wave,
                                                const int (&cp_off)[9]) {
    const uint8_t* gsrc = half_src + wave * 8 * kRowBytes;
    const uint32_t gdst = slot_addr + wave * 9 * 1024;
#pragma unroll
    for (int j = 0; j < 9; ++j) dma16(gdst + j * 1024, gsrc, (uint32_t)cp_off[j]);
}

// Wait until at most `ahead` half pages of this wave's copies are still in flight.
__device__ __forceinline__ void wait_copies(int ahead) {
    if (ahead >= 2) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if (ahead == 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier for LDS traffic only (outstanding copies stay in flight).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_bf16_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlotBytes];
    __shared__ __attribute__((aligned(16))) f32x4 xs[4 * 4 * 64];     // [wave][quarter][lane]

    const WorkItem w = p.work[blockIdx.x];
    if (w.b < 0) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = wave >> 1;     // which 32 rows of the tile
    const int h = wave & 1;         // which half of the dims (QK contraction and PV output)
    const int G = lane >> 5;        // MFMA k-group of this lane (0/1)
    const int lr = lane & 31;       // query row of this lane within the pair's 32
    const int b = w.b;
    const int n = min(max(p.seq_lens[b], 0), p.max_pages * kPage);
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    const uint8_t* kvbase = (const uint8_t*)p.kv;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_u8*)ring;

    // half pages of this unit that hold at least one token
    const int half_begin = 2 * w.page_begin;
    const int half_end = min(2 * w.page_end, (n + kHalfTok - 1) / kHalfTok);

    // per-lane copy offsets within an 8-token group
    int cp_off[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        const int qc = j * 64 + lane;
        const int t = qc / kRowChunks;
        const int pc = qc - t * kRowChunks;
        cp_off[j] = t * kRowBytes + ((pc ^ swz(t)) << 4);
    }
    // Page ids: lane i holds block-table entry page_begin + 64 g + i of the
    // current group g (bt_cur) and of group g + 1 (bt_nxt, loaded a group
    // ahead), so a copy never waits for a block-table load.
    int bt_grp = 0;
    auto bt_load = [&](int g) {
        const int pg = w.page_begin + 64 * g + lane;
        return pg < w.page_end ? bt[pg] : 0;
    };
    int bt_cur = bt_load(0);
    int bt_nxt = bt_load(1);
    auto half_src = [&](int k) {
        const int rel = (k >> 1) - w.page_begin;
        while ((rel >> 6) > bt_grp) {       // entering the next group of 64 pages
            bt_cur = bt_nxt;
            ++bt_grp;
            bt_nxt = bt_load(bt_grp + 1);
        }
        const int pid = __builtin_amdgcn_readlane(bt_cur, rel & 63);
        return kvbase + (size_t)pid * kPageBytes + (k & 1) * kSlotBytes;
    };
    // prologue: three half pages in flight before the query loads
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (half_begin + j < half_end)
            issue_half_copy(ring_addr + j * kSlotBytes, half_src(half_begin + j), wave, cp_off);

    // this lane's query row, its visible length, and its Q^T fragments:
    // k-step ks covers dims 288 h + 16 ks .. + 15, lane holds dims + 8 G .. + 7
    const int row = w.mt * kMTile + pair * 32 + lr;
    const bool row_ok = row < p.rows;
    const int tq = row / p.heads;
    const int nvis = p.causal ? max(n - (p.q_len - 1 - tq), 0) : n;
    // smallest visible length over every row of the workgroup: half pages below
    // it need no masking (row tiles span at most q_len query tokens)
    const int nvis_min = p.causal ? max(n - (p.q_len - 1), 0) : n;
    bf16x8_t qf[18];
    {
        const __bf16* qr = (const __bf16*)p.q + ((size_t)b * p.rows + (row_ok ? row : 0)) * kQK + 288 * h + 8 * G;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            bf16x8_t v = *(const bf16x8_t*)(qr + 16 * ks);
            qf[ks] = row_ok ? v : (bf16x8_t)0;
        }
    }

    // LDS read offsets within a slot.  QK: token lr, chunk c(ks) = 36 h + 2 ks + G
    // at position (c & ~7) | ((c ^ swz(lr)) & 7); c(ks + 4) = c(ks) + 8, so four
    // bases cover all 18 k-steps with immediate offsets 128 (ks / 4).
    int qk_off[4];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        const int c = 36 * h + 2 * k4 + G;
        qk_off[k4] = lr * kRowBytes + (((c & ~7) | ((c ^ swz(lr)) & 7)) << 4);
    }
    // PV transpose reads.  The 16-lane block bk = lane / 16 covers dims
    // 16 (bk % 2) .. + 15 of a 32-dim tile and tokens 16 k2 + 4 G + e (first
    // read) and + 8 (second read), e = (lane % 16) / 4; the lane supplies dims
    // 4 (lane % 4) .. + 3 of its token.  Dim tile dt of half h starts at dim
    // 256 h + 32 dt: chunk 32 h + 4 dt + 2 (bk % 2) + (lane % 4) / 2, and every
    // token read has swizzle 2 e + G.
    int tr_off[2];
    {
        const int li = lane & 15, e = li >> 2, cc = li & 3, dh = (lane >> 4) & 1;
        const int t = 4 * G + e;
        const int sw = swz(t);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
            tr_off[d2] = t * kRowBytes + h * 512 + (((4 * d2 + 2 * dh + (cc >> 1)) ^ sw) << 4) + (cc & 1) * 8;
    }
    __attribute__((address_space(3))) f32x4* xs_mine = (__attribute__((address_space(3))) f32x4*)xs + wave * 256 + lane;
    __attribute__((address_space(3))) f32x4* xs_other = (__attribute__((address_space(3))) f32x4*)xs + (wave ^ 1) * 256 + lane;

    f32x16 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        o[dt] = (f32x16)0.f;
        asm volatile("" : "+a"(o[dt]));
    }
    float m = -INFINITY, l = 0.f;

    auto slot_ptr = [&](int k) { return (lds_u8*)ring + ((k - half_begin) & 3) * kSlotBytes; };

    // Wait until half page k's copy has landed in every wave (and every wave
    // is past its previous use of the slot that the next refill targets).
    auto top = [&](int k) {
        wait_copies(min(2, half_end - 1 - k));
        lds_sync();
        const int tok0 = k * kHalfTok;
        if (tok0 + kHalfTok > n) {
            // rows past the sequence end may hold anything (NaN): zero them so
            // that a zero softmax weight times V stays zero
            lds_u8* cur = slot_ptr(k);
            const int t0 = n - tok0;
            for (int idx = threadIdx.x; idx < (kHalfTok - t0) * kRowChunks; idx += 256) {
                const int t = t0 + idx / kRowChunks;
                const int c = idx % kRowChunks;
                *(__attribute__((address_space(3))) i32x4*)(cur + t * kRowBytes + c * 16) = (i32x4)0;
            }
            lds_sync();
        }
    };
    // Partial S^T of half page k over this wave's 288 dims (two chains); K
    // fragments are read four k-steps ahead of their MFMA.
    auto qk = [&](int k, f32x16& sa, f32x16& sb) {
        lds_u8* cur = slot_ptr(k);
        sa = (f32x16)0.f;
        sb = (f32x16)0.f;
        auto kfrag = [&](int ks) -> bf16x8_t {
            return *(const __attribute__((address_space(3))) bf16x8_t*)(cur + qk_off[ks & 3] + (ks >> 2) * 128);
        };
        bf16x8_t kf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[ks] = kfrag(ks);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            const bf16x8_t a = kf[ks & 3];
            if (ks + 4 < 18) kf[ks & 3] = kfrag(ks + 4);
            if (ks & 1) sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sb, 0, 0, 0);
            else        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sa, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < 14; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // O^T += V^T . P^T over half page k (2 k-steps of 16 tokens x 8 dim tiles).
    // The MFMAs are inline assembly, which the compiler does not move loads
    // across, so the V^T fragments are software-pipelined here explicitly:
    // four fragments (eight transpose reads) are in flight ahead of the MFMA.
    auto pv = [&](int k, const bf16x8_t (&pf)[2]) {
        lds_u8* cur = slot_ptr(k);
        auto vfrag = [&](int i) -> bf16x8_t {      // i = 8 k2 + dt
            const int k2 = i >> 3, dt = i & 7;
            const int off = tr_off[dt & 1] + (dt >> 1) * 128 + k2 * 16 * kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(cur + off));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(cur + off + 8 * kRowBytes));
            return __builtin_bit_cast(bf16x8_t, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        };
        bf16x8_t vf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[i] = vfrag(i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // issued as inline assembly with O tied to its accumulation
            // registers, so the compiler never renames (and copies) O.  The
            // compiler does not see an MFMA here, so the wait states between a
            // VALU write of an operand (the P^T fragment, any register move of
            // the V^T fragment) and the MFMA read are inserted explicitly:
            // s_nop 3 gives 4.
            asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+a"(o[i & 7]) : "v"(vf[i & 3]), "v"(pf[i >> 3]));
            if (i + 4 < 16) vf[i & 3] = vfrag(i + 4);
        }
    };
    // MFMA results of the inline-assembly PV read by VALU code: the compiler
    // does not see those MFMAs, so the wait states are inserted here
    // (more than the 8-pass XDL write -> VALU / accvgpr read requirement).
    auto pv_drain = [&]() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); };
    // Pair sum of the partial tiles, masking of invisible tokens; returns the
    // row max in log2 units (logits stay unscaled: scale is applied in the
    // exponent, and scale > 0 commutes with the max).
    auto finish_s = [&](int k, const f32x16& sa, const f32x16& sb, f32x16& s) -> float {
        s = sa + sb;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            xs_mine[q4 * 64] = (f32x4){s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
        lds_sync();
        // every wave is past its reads of half page k - 1: refill its slot
        if (k + 3 < half_end)
            issue_half_copy(ring_addr + ((k + 3 - half_begin) & 3) * kSlotBytes, half_src(k + 3), wave, cp_off);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = xs_other[q4 * 64];
#pragma unroll
            for (int i = 0; i < 4; ++i) s[4 * q4 + i] += v[i];
        }
        // element i is token 32 k + 8 (i / 4) + 4 G + i % 4
        const int tok0 = k * kHalfTok;
        if (tok0 + kHalfTok > nvis_min) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = tok0 + 8 * (i >> 2) + 4 * G + (i & 3);
                s[i] = j < nvis ? s[i] : -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        return mx * p.scale_log2;
    };
    // Weights of half page k against the reference max m (log2 units); adds
    // the row sums.  exp2(c s - m) with c = scale * log2(e) is one FMA and one
    // exp; masked logits are -inf and give 0.
    auto weights = [&](f32x16& s, bf16x8_t (&pf)[2]) {
        const float c = p.scale_log2;
        const float mneg = m == -INFINITY ? 0.f : -m;
        float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, mneg));
            if (i & 1) sum1 += s[i]; else sum0 += s[i];
        }
        l += sum0 + sum1;
        // P^T fragments: k-step k2 (16 tokens) = accumulator elements 8 k2 .. + 7
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pf[0][e] = (__bf16)s[e];
            pf[1][e] = (__bf16)s[8 + e];
        }
    };

    // Software pipeline: the QK^T of half page k + 1 is issued together with
    // the PV of half page k.  The reference max m only moves when a row max
    // exceeds it by more than 2^8 (weights stay <= 2^8); that rescale of O
    // runs outside the inner loop, which never touches O with VALU work.
    if (half_begin < half_end) {
        int k = half_begin;
        f32x16 s, sa, sb;
        top(k);
        qk(k, sa, sb);
        float mx = finish_s(k, sa, sb, s);
        bool grow = mx > m + kRescaleSlack;
        for (;;) {
            if (__any(grow)) {
                pv_drain();
                const float m_new = grow ? mx : m;
                const float alpha = grow ? (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new)) : 1.f;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
                m = m_new;
            }
            bool done = false;
            for (;;) {
                bf16x8_t pf[2];
                const bool more = k + 1 < half_end;
                if (more) {
                    top(k + 1);
                    qk(k + 1, sa, sb);        // MFMAs run while the weights of k are computed
                }
                weights(s, pf);
                pv(k, pf);                    // PV MFMAs run through the pair exchange of k + 1
                if (!more) {
                    done = true;
                    break;
                }
                ++k;
                mx = finish_s(k, sa, sb, s);
                grow = mx > m + kRescaleSlack;
                if (__any(grow)) break;
            }
            if (done) break;
        }
    }

    pv_drain();
    // ---- epilogue: o = O / l, lse = ln(sum exp).  Both waves of a pair hold
    //      the full row sum; the lane pair (G = 0, 1) splits its tokens.
    const float lt = l + __shfl_xor(l, 32);
    if (!row_ok) return;
    const bool empty = m == -INFINITY;
    const float inv = empty ? 0.f : 1.f / lt;
    const float lse = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
    const int rit = row - w.mt * kMTile;
    // element i of dim tile dt is dim 256 h + 32 dt + 8 (i / 4) + 4 G + i % 4
    const int dim0 = 256 * h + 4 * G;
    if (w.nsplit == 1) {
        const size_t orow = (size_t)b * p.rows + row;
        if (p.out_bf16) {
            __bf16* dst = (__bf16*)p.out + orow * kV + dim0;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    __bf16 __attribute__((ext_vector_type(4))) v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[dt][4 * q4 + i] * inv);
                    *(__bf16 __attribute__((ext_vector_type(4)))*)(dst + 32 * dt + 8 * q4) = v;
                }
        } else {
            float* dst = (float*)p.out + orow * kV + dim0;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *(f32x4*)(dst + 32 * dt + 8 * q4) =
                        (f32x4){o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]} * inv;
        }
        if (G == 0 && h == 0) p.lse[orow] = lse;
    } else {
        float* dst = p.ws_o + ((size_t)blockIdx.x * kMTile + rit) * kV + dim0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(f32x4*)(dst + 32 * dt + 8 * q4) =
                    (f32x4){o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]} * inv;
        if (G == 0 && h == 0) p.ws_lse[(size_t)blockIdx.x * kMTile + rit] = lse;
    }
}

// ---------------------------------------------------------------------------
// LSE merge of one row from n partials: one wave, 8 output dims per lane
// ---------------------------------------------------------------------------
template <typename PartialAt>
__device__ __forceinline__ void merge_row(int n, PartialAt at, void* out, float* lse_out, size_t orow,
                                          int out_bf16) {
    const int lane = threadIdx.x & 63;
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, *at.lse(i));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    f32x4 acc0 = (f32x4)0.f, acc1 = (f32x4)0.f;
    float wsum = 0.f;
    if (mx != -INFINITY) {
        for (int i = 0; i < n; ++i) {
            const float li = *at.lse(i);
            if (li == -INFINITY) continue;
            const float wgt = __expf(li - mx);
            wsum += wgt;
            const f32x4* src = (const f32x4*)at.out(i) + 2 * lane;
            acc0 += wgt * src[0];
            acc1 += wgt * src[1];
        }
    }
    const bool empty = mx == -INFINITY;
    const float inv = empty ? 0.f : 1.f / wsum;
    acc0 *= inv;
    acc1 *= inv;
    if (out_bf16) {
        __bf16* dst = (__bf16*)out + orow * kV + 8 * lane;
        bf16x8 v;
        for (int i = 0; i < 4; ++i) { v[i] = (__bf16)acc0[i]; v[4 + i] = (__bf16)acc1[i]; }
        *(bf16x8*)dst = v;
    } else {
        f32x4* dst = (f32x4*)((float*)out + orow * kV) + 2 * lane;
        dst[0] = acc0;
        dst[1] = acc1;
    }
    if (lane == 0) lse_out[orow] = empty ? -INFINITY : mx + __logf(wsum);
}

struct SplitPartials {
    const float* ws_o;
    const float* ws_lse;
    int base, mt, m_tiles, rit;
    __device__ const float* lse(int s) const {
        return ws_lse + (size_t)unit_index(base + s, mt, m_tiles) * kMTile + rit;
    }
    __device__ const float* out(int s) const {
        return ws_o + ((size_t)unit_index(base + s, mt, m_tiles) * kMTile + rit) * kV;
    }
};

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const long long grow = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (grow >= (long long)p.batch * p.rows) return;
    const int b = (int)(grow / p.rows);
    const int r = (int)(grow - (long long)b * p.rows);
    const int S = p.req_info[2 * b];
    if (S <= 1) return;   // a single split wrote the result directly
    SplitPartials at{p.ws_o, p.ws_lse, p.req_info[2 * b + 1], r / kMTile, p.m_tiles, r % kMTile};
    merge_row(S, at, p.out, p.lse, (size_t)grow, p.out_bf16);
}

struct StackedPartials {
    const float* outs;
    const float* lses;
    size_t rows, row;
    __device__ const float* lse(int i) const { return lses + (size_t)i * rows + row; }
    __device__ const float* out(int i) const { return outs + ((size_t)i * rows + row) * kV; }
};

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    StackedPartials at{p.outs, p.lses, (size_t)p.rows, (size_t)row};
    merge_row(p.n, at, p.out, p.lse, (size_t)row, p.out_bf16);
}

// ---------------------------------------------------------------------------
// launchers.  hipGetLastError() is read once before each launch so that a
// stale error left by an unrelated earlier HIP call is not reported as this
// launch's failure, and once after it for the launch's own status.
// ---------------------------------------------------------------------------
static inline void clear_stale_error() { (void)hipGetLastError(); }
hipError_t launch_plan(const PlanParams& p, const int32_t* seq_lens, int32_t* req_info,
                       WorkItem* work, hipStream_t stream) {
    clear_stale_error();
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p, seq_lens, req_info, work);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeParams& p, int units, hipStream_t stream,
                              hipEvent_t ev_before, hipEvent_t ev_after) {
    if (ev_before) {
        hipError_t e = hipEventRecord(ev_before, stream);
        if (e != hipSuccess) return e;
    }
    clear_stale_error();
    hipLaunchKernelGGL(decode_bf16_kernel, dim3(units), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_after) return hipEventRecord(ev_after, stream);
    return hipSuccess;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
    const long long rows = (long long)p.batch * p.rows;
    if (rows == 0) return hipSuccess;
    clear_stale_error();
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    clear_stale_error();
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
