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
//   decode_fp8      - the same for an OCP fp8 e4m3 cache and query (fp8 MFMA for both products)
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
// within aligned groups of 8 by c -> c ^ swz(t).  gfx950's LDS has 64 banks of
// 4 bytes and serves a 16-byte-per-lane read 16 lanes (256 bytes) at a time.
// A 1152-byte row stride moves the bank window by 128 bytes per token, so
// tokens of one parity share their window offset: swz is 16-periodic and gives
// the 8 even and the 8 odd tokens of any 16 distinct values (row-fragment reads
// of 16 tokens x 16 B hit all 64 banks once; with an 8-periodic swizzle tokens
// t and t + 8 collide), and keeps bit 2 different between tokens 4j + i and
// 4j + i + 2 (transpose reads of 4 tokens x 4 chunks hit distinct banks).
// swz(t + 8) = swz(t) ^ 2 and swz(t + 16) = swz(t).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int t) { return (((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2); }

// ---------------------------------------------------------------------------
// split planner: per-request split counts, first kv-units and work items,
// from seq_lens on the device (no host sync).  plan_splits runs on one block
// of NT threads over LDS scratch the caller provides.  plan_kernel runs it
// once (one 1024-thread workgroup) and writes the whole work list; for small
// batches every decode workgroup runs it itself, in its still empty LDS ring,
// and keeps only its own item (no separate launch).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) int lds_int;
typedef __attribute__((address_space(3))) unsigned int lds_uint;

// Wave-wide inclusive prefix sum / running max through DPP (row shifts within
// each 16-lane row, then the row broadcasts of lanes 15 and 31): six VALU
// steps, where shuffles through the LDS crossbar would each take a round trip.
// Lane 63 ends with the whole wave's sum / max.
__device__ __forceinline__ int wave_scan_add(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return v;
}
__device__ __forceinline__ int wave_scan_max(int v) {   // v >= 0
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
    return v;
}
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_scan_add(v), 63); }

struct PlanScratch {
    lds_int* pages;      // [cached] page counts
    lds_int* first;      // [cached] first piece of each request
    lds_int* gstart;     // [cached] first global page of each request (balanced plan)
    lds_int* part;       // [3][waves] per-wave page sums (16-bit halves) and longest request
    lds_uint* cnt;       // [2][16] kv-units per candidate chunk, two rounds in turn
    lds_int* scan;       // [2][waves] wave totals of the two scans
    lds_int* owner;      // [4] the probed slot's request, its split or first page, first piece, pieces
    lds_int* hist;       // [256] requests starting inside each kv-unit (balanced plan)
    int cached;          // requests whose page count, first piece and first page stay in LDS
};

constexpr int kPieceCostPages = 2;   // a piece's fixed cost (pipeline fill, epilogue), in pages

struct PlanResult {
    int chunk;           // pages per split (common-chunk plan)
    int k_total;         // kv-units in all
    int balanced;        // > 0: the balanced plan, with this many pages per kv-unit
    int total_pages;     // all requests' pages (balanced plan)
    int group;           // kv-units per work item: consecutive splits of one request (>= 1)
};

// Forced splits (num_splits > 0) that cut every request into the same number
// S of splits and make more work items than one round of workgroups: each
// item takes `group` consecutive splits of one request (the smallest divisor
// of S that brings the items within one round), so that a workgroup pays its
// fixed cost (query tile, planning) once per group.  Only when the caller
// launches a kernel instance that runs groups (PlanParams::group_ok).
__device__ __forceinline__ int split_group(const PlanParams& p, int k_total, int longest) {
    if (!p.group_ok || p.num_splits <= 0 || p.balance || p.batch <= 0) return 1;
    const int S = min(p.num_splits, max(longest, 1));
    if ((long long)k_total != (long long)p.batch * S) return 1;   // some request has fewer splits
    const long long items = (long long)k_total * p.m_tiles;
    const long long cap = p.target_units > 0 ? p.target_units : 1;
    if (items <= cap) return 1;
    const int need = (int)min((items + cap - 1) / cap, (long long)S);
    for (int g = need; g < S; ++g)
        if (S % g == 0) return g;
    return S;
}

// Runs on all NT threads of the block (every barrier inside is reached by all
// of them); req_info, if not null, receives the kReqInfoInts values per
// request.  probe_slot >= 0 names a work slot whose request the thread that
// owns the request describes in L.owner (see plan_item).
//
// Two plans.  Common chunk: request b of P_b pages is cut into splits of c
// pages (the smallest c that fits every request's splits into one round of
// workgroups), one kv-unit per split.  Balanced: when that plan's longest
// kv-unit is more than 1/8 above the average, the pages of all requests are
// laid end to end and cut into kv-units of C = ceil(sum P / U) pages; a
// kv-unit then holds one piece of every request it touches.
template <int NT>
__device__ __forceinline__ PlanResult plan_splits(const PlanParams& p, const int32_t* __restrict__ seq_lens,
                                                  const PlanScratch& L, int32_t* __restrict__ req_info,
                                                  int probe_slot = -1) {
    constexpr int kWaves = NT / 64;
    constexpr int kCand = 16;                // chunk sizes counted per round
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int per = (p.batch + NT - 1) / NT;
    const int b0 = min(p.batch, tid * per), b1 = min(p.batch, b0 + per);
    const int cap = p.max_pages * kPage;
    auto pages_global = [&](int b) {
        const int n = min(max(seq_lens[b], 0), cap);
        return (n + kPage - 1) / kPage;
    };
    // page counts into LDS, with the total and the longest request on the way.
    // A lane's sum can pass 2^31 only in theory (2^20 requests of 2^24 pages),
    // so the total travels as two 16-bit halves, each summed in 32 bits.
    unsigned long long my_total = 0;
    int my_longest = 0;
    for (int b = tid; b < p.batch; b += NT) {
        const int pg = pages_global(b);
        if (b < L.cached) L.pages[b] = pg;
        my_total += (unsigned long long)pg;
        my_longest = max(my_longest, pg);
    }
    const int t_lo = wave_sum((int)(my_total & 0xffff));
    const int t_hi = wave_sum((int)(my_total >> 16));
    const int w_longest = __builtin_amdgcn_readlane(wave_scan_max(my_longest), 63);
    if (lane == 0) {
        L.part[wv] = t_lo;
        L.part[kWaves + wv] = t_hi;
        L.part[2 * kWaves + wv] = w_longest;
    }
    __syncthreads();
    auto pages_of = [&](int b) { return b < L.cached ? L.pages[b] : pages_global(b); };
    unsigned long long total_pages = 0;
    int longest = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        total_pages += (unsigned long long)(unsigned)L.part[i] + ((unsigned long long)(unsigned)L.part[kWaves + i] << 16);
        longest = max(longest, L.part[2 * kWaves + i]);
    }

    int chunk = 1;
    int balanced = 0;
    if (p.num_splits <= 0) {
        // The smallest chunk (in pages) for which every request's splits, times
        // the row tiles, fit in one round of target_units workgroups: the
        // longest unit, and so the kernel, is then as short as this policy
        // allows.  It lies between the averaging bound and the longest request
        // (any chunk at or past the longest request gives every request one
        // split, the same work list); when even that does not fit, the longest
        // request is the chunk.  Each round counts 16 chunk sizes at once (the
        // waves share them out): first the 16 sizes from the averaging bound
        // up (the answer is almost always among them), then 16 sizes spread
        // evenly over what is left of the range, which shrinks it 16-fold.
        const long long units_cap = p.target_units / p.m_tiles > 0 ? p.target_units / p.m_tiles : 1;
        const long long avg = (long long)((total_pages + units_cap - 1) / units_cap);
        const int hi0 = max(longest, 1);
        int lo = (int)(avg < hi0 ? avg : hi0);
        lo = lo > p.min_chunk ? lo : min(p.min_chunk, hi0);
        int hi = hi0;
        // kv-units at chunk c >= avg: at most units_cap + batch, so 32 bits hold them
        auto count = [&](int c) {
            unsigned int cnt = 0;
            for (int b = lane; b < p.batch; b += 64) {
                const unsigned int pg = (unsigned int)pages_of(b);
                cnt += pg > (unsigned int)c ? (pg + c - 1) / (unsigned int)c : 1u;
            }
            return (unsigned int)wave_sum((int)cnt);
        };
        // invariant: the answer is the smallest fitting chunk in [lo, hi], or hi if none fits
        for (int round = 0;; ++round) {
            const bool dense = round == 0 || hi - lo < kCand;
            auto cand = [&](int j) {
                return dense ? min(lo + j, hi) : lo + (int)((long long)(hi - lo) * (j + 1) / kCand);
            };
            lds_uint* cnt = L.cnt + (round & 1) * kCand;
#pragma unroll
            for (int j = wv; j < kCand; j += kWaves) {
                const unsigned int mine = count(cand(j));
                if (lane == 0) cnt[j] = mine;
            }
            __syncthreads();
            int first = -1;   // first candidate that fits
            for (int j = kCand - 1; j >= 0; --j)
                if ((long long)cnt[j] <= units_cap) first = j;
            if (dense && (hi - lo < kCand || first >= 0)) {
                chunk = first >= 0 ? cand(first) : hi;
                break;
            }
            if (first < 0) {
                if (dense) {
                    lo += kCand;          // lo .. lo + 15 do not fit; go on above them
                    continue;
                }
                chunk = hi;               // hi itself was counted and does not fit
                break;
            }
            lo = first > 0 ? cand(first - 1) + 1 : lo;
            hi = cand(first);
        }
        // a candidate for the balanced plan: the common chunk fits one round
        // but leaves the longest kv-unit more than 1/8 above the averaging
        // bound (global page indices stay below 2^30)
        const int c_avg = max((int)min(avg, (long long)INT32_MAX), p.min_chunk);
        if (p.balance && total_pages > 0 && total_pages < (1ull << 30) && chunk > c_avg + max(1, c_avg / 8) &&
            (long long)count(chunk) <= units_cap)
            balanced = c_avg;
    }

    // first global page of each request (balanced plan): exclusive scan of
    // the page counts (a wavefront scan, then the wave totals through LDS)
    int my_g = 0;
    if (balanced) {
        int my_pages = 0;
        for (int b = b0; b < b1; ++b) my_pages += pages_of(b);
        const int incl = wave_scan_add(my_pages);
        if (lane == 63) L.scan[wv] = incl;
        __syncthreads();
        int wave_base = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) wave_base += i < wv ? L.scan[i] : 0;
        my_g = wave_base + incl - my_pages;
        // Each piece costs a pipeline fill and an epilogue besides its pages
        // (about kPieceCostPages pages' time): the balanced plan is kept only
        // if its busiest kv-unit, with one extra piece per request starting
        // inside it, still beats the common chunk by 1/8.
        const int A = balanced;
        const int k_bal = (int)((total_pages + A - 1) / A);
        for (int i = tid; i < k_bal; i += NT) L.hist[i] = 0;
        __syncthreads();
        int g = my_g;
        for (int b = b0; b < b1; ++b) {
            const int pages = pages_of(b);
            if (pages > 0 && g % A != 0) atomicAdd((int*)(L.hist + g / A), 1);
            g += pages;
        }
        __syncthreads();
        int my_max = 0;
        for (int i = tid; i < k_bal; i += NT) my_max = max(my_max, (int)L.hist[i]);
        const int w_max = __builtin_amdgcn_readlane(wave_scan_max(my_max), 63);
        if (lane == 0) L.scan[wv] = w_max;
        __syncthreads();
        int max_extra = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) max_extra = max(max_extra, (int)L.scan[i]);
        if (A + kPieceCostPages * max_extra + max(1, A / 8) >= chunk) balanced = 0;
        __syncthreads();   // L.scan is reused below
    }
    // pieces per request: splits (common chunk); kv-units touched, none for
    // an empty request (balanced)
    auto pieces_of = [&](int pages, int g) {
        if (balanced) return pages > 0 ? (g + pages - 1) / balanced - g / balanced + 1 : 0;
        const int S = p.num_splits > 0 ? min(p.num_splits, pages) : (pages + chunk - 1) / chunk;
        return max(S, 1);
    };
    int my_k = 0;
    {
        int g = my_g;
        for (int b = b0; b < b1; ++b) {
            const int pages = pages_of(b);
            my_k += pieces_of(pages, g);
            g += pages;
        }
    }
    const int incl = wave_scan_add(my_k);
    if (lane == 63) L.scan[kWaves + wv] = incl;
    if (probe_slot >= 0 && tid == 0) L.owner[0] = -1;   // (set below by the owning thread)
    __syncthreads();
    int wave_base = 0, pieces_total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = L.scan[kWaves + i];
        wave_base += i < wv ? t : 0;
        pieces_total += t;
    }
    const int k_total = balanced ? (int)((total_pages + balanced - 1) / balanced) : pieces_total;
    const int group = balanced ? 1 : split_group(p, k_total, longest);
    // the probed slot's first kv-unit (the layout of plan_item)
    int probe_k = -1;
    if (probe_slot >= 0) {
        const int items = k_total / group;
        const int per_xcd = (items + 7) / 8;
        const int kx = (probe_slot >> 3) / p.m_tiles;
        probe_k = kx < per_xcd ? per_xcd * (probe_slot & 7) + kx : -1;
        probe_k = probe_k >= 0 && probe_k < items ? probe_k * group : -1;
    }
    int base = wave_base + incl - my_k;
    int g = my_g;
    for (int b = b0; b < b1; ++b) {
        const int pages = pages_of(b);
        const int S = pieces_of(pages, g);
        if (req_info) {
            req_info[kReqInfoInts * b] = S;
            req_info[kReqInfoInts * b + 1] = base;
            req_info[kReqInfoInts * b + 2] = balanced ? g : 0;
            req_info[kReqInfoInts * b + 3] = 0;
        }
        if (b < L.cached) {
            L.first[b] = base;
            L.gstart[b] = g;
        }
        if (probe_k >= 0) {
            // the request holding kv-unit probe_k (common chunk), or the one
            // holding its first page (balanced)
            const bool mine = balanced ? (pages > 0 && (long long)probe_k * balanced >= g &&
                                          (long long)probe_k * balanced < g + pages)
                                       : (probe_k >= base && probe_k < base + S);
            if (mine) {
                L.owner[0] = b;
                L.owner[1] = balanced ? g : probe_k - base;
                L.owner[2] = base;
                L.owner[3] = S;
            }
        }
        base += S;
        g += pages;
    }
    __syncthreads();   // first pieces and pages of every cached request visible to the block
    return PlanResult{chunk, k_total, balanced, balanced ? (int)total_pages : 0, group};
}

// Slot u's first kv-unit and row tile.  Dispatch deals workgroups to the 8
// XCDs round-robin, so slot u runs on XCD u % 8 as its (u / 8)-th workgroup
// there.  Each XCD takes a contiguous run of C = ceil(items / 8) work items
// (an item is `group` consecutive kv-units) with all their row tiles: slot u
// holds item q = C (u % 8) + (u / 8) / m_tiles, i.e. kv-unit k = q group, and
// row tile (u / 8) % m_tiles.  The splits of one request (which read the same
// query rows) and the row tiles of one kv-unit (which read the same pages)
// then share one L2.  Returns false for an empty slot.
__device__ __forceinline__ bool slot_unit(const PlanParams& p, const PlanResult& r, int u, int& k, int& mt) {
    const int items = r.k_total / r.group;
    const int per_xcd = (items + 7) / 8;
    const int pos = u >> 3;
    const int kx = pos / p.m_tiles;
    const int q = per_xcd * (u & 7) + kx;
    k = q * r.group;
    mt = pos - kx * p.m_tiles;
    return kx < per_xcd && q < items;
}

__device__ __forceinline__ WorkItem empty_item() {
    WorkItem w;
    w.b = -1; w.mt = 0; w.piece = 0; w.page_begin = 0; w.npages = 0; w.nsplit = 0; w.g0 = 0; w.chunk = 0;
    return w;
}

// The work item of kv-unit k, row tile mt, whose first request b has `pages`
// pages, first piece `first`, S pieces and (balanced plan) first global page g
// (common chunk: `split_or_g` is the split index instead).
__device__ __forceinline__ WorkItem make_item(const PlanParams& p, const PlanResult& r, int k, int mt, int b,
                                              int pages, int split_or_g, int first, int S) {
    WorkItem w;
    w.b = b;
    w.mt = mt;
    w.nsplit = S;
    if (r.balanced) {
        const int C = r.balanced;
        const int g0 = k * C;
        w.piece = first + (k - split_or_g / C);
        w.page_begin = g0 - split_or_g;
        w.npages = min(g0 + C, r.total_pages) - g0;
        w.g0 = g0;
        w.chunk = C;
    } else {
        // (a group of splits: g0 = their count, each of cb pages but the last)
        const int cb = p.num_splits > 0 ? (pages + S - 1) / S : r.chunk;
        const int pb = min(pages, split_or_g * cb);
        w.piece = k;
        w.page_begin = pb;
        w.npages = min(pages, (split_or_g + r.group) * cb) - pb;
        w.g0 = r.group > 1 ? r.group : 0;
        w.chunk = 0;
    }
    return w;
}

// Work item of slot u for the planner kernel: the request of kv-unit k by
// binary search over the first pieces (common chunk) or first pages
// (balanced: the last request starting at or before the unit's first page
// is the non-empty one holding it).
template <typename FirstOf, typename GstartOf, typename PagesOf>
__device__ __forceinline__ WorkItem plan_item(const PlanParams& p, const PlanResult& r, int u,
                                              FirstOf&& first_of, GstartOf&& gstart_of, PagesOf&& pages_of) {
    int k, mt;
    if (!slot_unit(p, r, u, k, mt)) return empty_item();
    const long long key = r.balanced ? (long long)k * r.balanced : k;
    int lo = 0, hi = p.batch - 1;     // last request whose first piece / page is <= key
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((r.balanced ? gstart_of(mid) : first_of(mid)) <= key) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int first = first_of(b);
    if (r.balanced) {
        const int pg = pages_of(b), g = gstart_of(b);
        const int S = pg > 0 ? (g + pg - 1) / r.balanced - g / r.balanced + 1 : 0;
        return make_item(p, r, k, mt, b, pg, g, first, S);
    }
    const int S = (b + 1 < p.batch ? first_of(b + 1) : r.k_total) - first;
    return make_item(p, r, k, mt, b, pages_of(b), k - first, first, S);
}

__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p, const int32_t* __restrict__ seq_lens,
                                                    int32_t* __restrict__ req_info,
                                                    WorkItem* __restrict__ work) {
    constexpr int kCached = 8192;            // requests whose values stay in LDS
    __shared__ int s_pages[kCached];
    __shared__ int s_first[kCached];
    __shared__ int s_gstart[kCached];
    __shared__ int s_part[48];
    __shared__ unsigned int s_cnt[32];
    __shared__ int s_scan[32];
    __shared__ int s_hist[256];
    const PlanScratch L{(lds_int*)s_pages, (lds_int*)s_first, (lds_int*)s_gstart, (lds_int*)s_part,
                        (lds_uint*)s_cnt, (lds_int*)s_scan, nullptr, (lds_int*)s_hist, kCached};
    const PlanResult r = plan_splits<1024>(p, seq_lens, L, req_info);
    const int cap = p.max_pages * kPage;
    auto pages_of = [&](int b) {
        if (b < kCached) return s_pages[b];
        const int n = min(max(seq_lens[b], 0), cap);
        return (n + kPage - 1) / kPage;
    };
    auto first_of = [&](int b) { return b < kCached ? s_first[b] : req_info[kReqInfoInts * b + 1]; };
    auto gstart_of = [&](int b) { return b < kCached ? s_gstart[b] : req_info[kReqInfoInts * b + 2]; };
    for (int u = threadIdx.x; u < p.units_max; u += 1024)
        work[u] = plan_item(p, r, u, first_of, gstart_of, pages_of);
}

// The decode kernels' own copy of the planner for batches of at most
// kFusedPlanMax requests, in the first bytes of their LDS ring (before any
// copy into it).  Every workgroup derives the same plan and keeps its own
// item, which it also stores to the work list; workgroup 0 stores the
// per-request values the combine reads.  The item is the same value in every
// lane; readfirstlane makes that visible to the compiler.
template <int NT>
__device__ __forceinline__ WorkItem decode_work_item(const DecodeParams& p, uint8_t* lds) {
    static_assert(NT % 64 == 0 && NT <= 1024, "whole waves, at most 16");
    if (!p.fused_plan) {
        // A stored work list may come from an earlier planner run: an item
        // that does not fit this call's descriptor (a list planned for
        // another one, or never written) is skipped rather than followed.
        WorkItem w = p.work[blockIdx.x];
        if (w.b >= p.plan.batch || w.mt < 0 || w.mt >= p.plan.m_tiles || w.page_begin < 0 || w.npages < 0 ||
            w.page_begin > p.max_pages || w.npages > (w.chunk > 0 ? w.chunk : p.max_pages) || w.nsplit < 1 ||
            w.piece < 0 || w.chunk < 0 || w.g0 < 0 ||
            (w.chunk == 0 && w.g0 > 1 && (!p.plan.group_ok || w.g0 > w.nsplit)))
            w.b = -1;
        return w;
    }
    lds_u8* l8 = (lds_u8*)lds;
    // scratch after the page counts, first pieces and first pages: per-wave
    // sums [3][16], candidate counts [2][16], scan totals [2][16], the probed
    // slot's owner [4], kv-unit histogram [256]
    constexpr int kOff = 12 * kFusedPlanMax;
    const PlanScratch L{(lds_int*)l8, (lds_int*)(l8 + 4 * kFusedPlanMax), (lds_int*)(l8 + 8 * kFusedPlanMax),
                        (lds_int*)(l8 + kOff), (lds_uint*)(l8 + kOff + 192), (lds_int*)(l8 + kOff + 320),
                        (lds_int*)(l8 + kOff + 448), (lds_int*)(l8 + kOff + 512), kFusedPlanMax};
    const int u = blockIdx.x;
    const PlanResult r = plan_splits<NT>(p.plan, p.seq_lens, L, u == 0 ? p.req_info : nullptr, u);
    // this slot's item, its request described by the thread that owns it
    int k, mt;
    WorkItem w = empty_item();
    if (slot_unit(p.plan, r, u, k, mt) && L.owner[0] >= 0) {
        const int b = L.owner[0];
        w = make_item(p.plan, r, k, mt, b, L.pages[b], L.owner[1], L.owner[2], L.owner[3]);
    }
    // the same value in every lane: say so, so that it stays in scalar registers
    w.b = __builtin_amdgcn_readfirstlane(w.b);
    w.mt = __builtin_amdgcn_readfirstlane(w.mt);
    w.piece = __builtin_amdgcn_readfirstlane(w.piece);
    w.page_begin = __builtin_amdgcn_readfirstlane(w.page_begin);
    w.npages = __builtin_amdgcn_readfirstlane(w.npages);
    w.nsplit = __builtin_amdgcn_readfirstlane(w.nsplit);
    w.g0 = __builtin_amdgcn_readfirstlane(w.g0);
    w.chunk = __builtin_amdgcn_readfirstlane(w.chunk);
    if (threadIdx.x == 0) p.work_out[u] = w;
    __syncthreads();   // the LDS ring is filled next
    return w;
}

// The one piece of an item that is neither a group nor a balanced range.
__device__ __forceinline__ Piece single_piece(const DecodeParams& p, const WorkItem& w) {
    const __attribute__((address_space(4))) int32_t* sl = (const __attribute__((address_space(4))) int32_t*)p.seq_lens;
    const int n = min(max(sl[w.b], 0), p.max_pages * kPage);
    Piece pc;
    pc.b = __builtin_amdgcn_readfirstlane(w.b);
    pc.mt = __builtin_amdgcn_readfirstlane(w.mt);
    pc.page_begin = __builtin_amdgcn_readfirstlane(w.page_begin);
    pc.page_end = __builtin_amdgcn_readfirstlane(min((n + kPage - 1) / kPage, w.page_begin + w.npages));
    pc.nsplit = __builtin_amdgcn_readfirstlane(w.nsplit);
    pc.slot = __builtin_amdgcn_readfirstlane(w.piece * p.plan.m_tiles + w.mt);
    pc.run = 1;
    pc.run_pages = 0;
    return pc;
}

// The piece of an item that is a group of consecutive forced splits of one
// request (chunk 0, g0 > 1 splits of ceil(pages / nsplit) pages each, the
// last ones possibly short or empty), as one run; splits whose partial slot
// would lie past the workspace are dropped.  Any other item: its single piece.
__device__ __forceinline__ Piece group_piece(const DecodeParams& p, const WorkItem& w) {
    if (!(w.chunk <= 0 && w.g0 > 1)) return single_piece(p, w);
    const __attribute__((address_space(4))) int32_t* sl = (const __attribute__((address_space(4))) int32_t*)p.seq_lens;
    const int n = min(max(sl[w.b], 0), p.max_pages * kPage);
    const int pages = (n + kPage - 1) / kPage;
    const int cb = max((pages + max(w.nsplit, 1) - 1) / max(w.nsplit, 1), 1);
    const int slot = w.piece * p.plan.m_tiles + w.mt;
    const int fit = slot < p.plan.units_max ? (p.plan.units_max - 1 - slot) / p.plan.m_tiles + 1 : 0;
    const int run = min(w.g0, fit);
    const int pb = min(pages, w.page_begin);
    Piece pc;
    pc.b = __builtin_amdgcn_readfirstlane(w.b);
    pc.mt = __builtin_amdgcn_readfirstlane(w.mt);
    pc.page_begin = __builtin_amdgcn_readfirstlane(pb);
    pc.page_end = __builtin_amdgcn_readfirstlane(max(pb, min(min(pages, w.page_begin + w.npages), w.page_begin + run * cb)));
    pc.nsplit = __builtin_amdgcn_readfirstlane(w.nsplit);
    pc.slot = __builtin_amdgcn_readfirstlane(slot);
    pc.run = __builtin_amdgcn_readfirstlane(run);
    pc.run_pages = __builtin_amdgcn_readfirstlane(cb);
    return pc;
}

// Runs body(piece) for each piece of work item w in turn (a barrier between
// pieces: every piece reuses the whole LDS).  Pieces after the first start at
// page 0 of the next non-empty request; the balanced plan's global page
// arithmetic gives each its piece count.
template <typename Body>
__device__ __forceinline__ void for_each_piece(const DecodeParams& p, const WorkItem& w, Body&& body) {
    const int cap = p.max_pages * kPage;
    // (the lengths through the scalar unit: the piece loop keeps no VGPR)
    const __attribute__((address_space(4))) int32_t* sl = (const __attribute__((address_space(4))) int32_t*)p.seq_lens;
    auto pages_of = [&](int b) {
        const int n = min(max(sl[b], 0), cap);
        return (n + kPage - 1) / kPage;
    };
    Piece pc;
    pc.b = w.b;
    pc.mt = w.mt;
    pc.page_begin = w.page_begin;
    pc.nsplit = w.nsplit;
    pc.run = 1;
    pc.run_pages = 0;
    int piece = w.piece;
    int left = w.npages, done = 0;
    for (;;) {
        pc.page_end = min(pages_of(pc.b), pc.page_begin + left);
        pc.slot = piece * p.plan.m_tiles + pc.mt;
        // (one value in every lane: kept in scalar registers)
        pc.b = __builtin_amdgcn_readfirstlane(pc.b);
        pc.mt = __builtin_amdgcn_readfirstlane(pc.mt);
        pc.page_begin = __builtin_amdgcn_readfirstlane(pc.page_begin);
        pc.page_end = __builtin_amdgcn_readfirstlane(pc.page_end);
        pc.nsplit = __builtin_amdgcn_readfirstlane(pc.nsplit);
        pc.slot = __builtin_amdgcn_readfirstlane(pc.slot);
        // (a stored item that points past the workspace's partial slots is not followed)
        if (pc.nsplit > 1 && (pc.slot < 0 || pc.slot >= p.plan.units_max)) break;
        body(pc);
        const int took = pc.page_end - pc.page_begin;
        left -= took;
        done += took;
        if (w.chunk <= 0 || left <= 0 || took <= 0) break;
        int b = pc.b + 1;
        while (b < p.plan.batch && pages_of(b) == 0) ++b;
        if (b >= p.plan.batch) break;
        __syncthreads();
        const int g = w.g0 + done;   // the request's first global page
        pc.b = __builtin_amdgcn_readfirstlane(b);
        pc.page_begin = 0;
        pc.nsplit = __builtin_amdgcn_readfirstlane((g + pages_of(b) - 1) / w.chunk - g / w.chunk + 1);
        ++piece;
    }
}

// ---------------------------------------------------------------------------
// split-KV decode, bf16 cache: shared layout and helpers
//
// kMTile = 128 query rows per work item (request, 128-row tile, page range),
// so every cache page is ingested once per 128 rows.  Both contractions run
// on v_mfma_f32_32x32x16_bf16 with the query rows as the MFMA N dimension:
//   S^T[32 tok][32 rows]  += K[32 tok][16 dims]  . Q^T[16 dims][32 rows]
//   O^T[32 dims][32 rows] += V^T[32 dims][16 tok] . P^T[16 tok][32 rows]
// The cache streams through LDS in half pages of 32 tokens (36,864 bytes)
// held in a ring of 4 slots, filled by direct HBM -> LDS loads three half
// pages ahead of the one being contracted.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kHalfTok = 32;                          // tokens per ring slot
constexpr int kSlotBytes = kHalfTok * kRowBytes;      // 36,864
constexpr int kSlots = 4;
constexpr int kRingBytes = kSlots * kSlotBytes;       // 147,456

// One direct HBM -> LDS load of 16 bytes per lane: lane i writes LDS bytes
// [lds_addr + 16 i, +16) with the 16 bytes at gbase + voff.  Issued as inline
// assembly so that the compiler does not track it: the caller waits for it
// explicitly before the data is read, and the compiler's own LDS waits stay
// exact instead of draining every pending LDS read.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* gbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8) that wait for vector memory only.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier for LDS traffic only (outstanding copies stay in flight).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max over the lane pair (l, l ^ 32) without LDS: the swap leaves both values of
// the pair in (r[0], r[1]) on both lanes.
__device__ __forceinline__ float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max of three floats in one v_max3_f32, without the quieting v_max x, x, x
// that fmaxf puts before values it cannot prove canonical
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The lane index, recomputed where it is called (mbcnt in inline assembly):
// the decode bodies run once per piece inside a loop, and a lane index the
// compiler may hoist would drag every value derived from it out of the loop,
// live (in VGPRs) across the whole body.
__device__ __forceinline__ int lane_id_fresh() {
    int v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

// ---------------------------------------------------------------------------
// split-KV decode, bf16 cache, two waves per SIMD with split roles
//
// Workgroup = 8 waves (two per SIMD) over one work item of kMTile = 128
// query rows.  One wave per SIMD can only read about 24 bytes
// of LDS per clock, while QK^T with Q resident in registers consumes a 1 KB
// K fragment per 32-clock MFMA; a second wave on each SIMD supplies MFMAs of
// its own while the first waits on LDS.  The register file decides the
// split: the 128 rows' O accumulators (256 KB) and query (147 KB) fill 79 % of
// the CU's 512 KB, so the two waves of a SIMD take different roles:
//  - wave A of SIMD s owns query rows 32 s .. 32 s + 31: their whole Q^T in
//    registers (144 VGPRs), QK^T over all 576 dims, the online softmax (exact
//    row max, reference max in whole log2 units), and publishes P^T of the
//    tile; it also accumulates O^T for dim tile 4 s (32 dims) of all four row
//    tiles (64 AGPRs);
//  - wave B of SIMD s accumulates O^T for dim tiles 4 s + 1 .. 4 s + 3 of all
//    four row tiles, and issues every page copy.  The split between VGPRs and
//    AGPRs is one per kernel and would be even, so no accumulator lives in an
//    AGPR: the MFMAs accumulate in VGPRs, and each wave has 256 of them.
// Each V^T fragment read from LDS feeds four MFMAs (one per row tile).  Per
// 32-token step a SIMD runs 36 + 8 MFMAs on wave A and 24 on wave B.
// Roles follow the hardware SIMD of each wave (HW_ID), read once: the lower
// wave index of a SIMD is A; if the SIMD ids do not come out two per SIMD,
// waves 0-3 are A and 4-7 B (same results, only the overlap differs).
//
// LDS: a 4-slot ring of half pages (147,456 bytes) and a double-buffered P^T
// exchange (2 x 8 KB): the whole 160 KB.  The reference max moves in whole
// log2 units, so every rescale factor is an exact power of two 2^-d; the
// k-step 0 fragment of a tile carries d in the sign bits of its weights
// (which are non-negative): element 0 flags a move, elements 1 .. 7 hold d.
//
// One step k, one barrier T(k): the copies of half page k + 1 have landed,
// P(k) is published, and every wave is past its PV of half page k - 1 (so B
// refills that slot with half page k + 3).  Then A: PV of k, QK^T and softmax
// of k + 1 (P(k + 1) into the other buffer); B: copies, PV of k.
// ---------------------------------------------------------------------------
constexpr int kAbPBufOff = kRingBytes;                 // [2 buffers][4 tiles][2 k-steps][64 lanes] 16 B
constexpr int kAbLdsBytes = kAbPBufOff + 2 * 8192;     // 163,840 (the whole LDS)
static_assert(kAbLdsBytes <= 163840, "LDS budget");
constexpr float kRescaleSlackAb = 8.f;                 // reference max moves when the max grows by > 2^8

// SIMD of the calling wave (HW_ID bits 5:4)
__device__ __forceinline__ int hw_simd_id() {
    return (int)(__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3u);
}

// The query tile of rows [mt kMTile, + kMTile) of request b through the still
// empty ring (rows swizzled like cache rows, 144 blocks of 1 KB, 18 per wave);
// then each A wave reads its rows' Q^T fragments: k-step ks covers dims 16 ks
// .. + 15, lane (lr, G) holds dims + 8 G .. + 7 of row lr (chunk 2 ks + G).
// All 8 waves take part (two barriers).  The splits of a group reuse the
// fragments (same request and rows).
template <bool A>
__device__ __forceinline__ void stage_query_bf16(const DecodeParams& p, int b, int mt, uint8_t* lds, int s, int wv,
                                                 bf16x8_t (&qf)[36]) {
    const int lane = lane_id_fresh();
    const int G = lane >> 5, lr = lane & 31;
    lds_u8* const ring = (lds_u8*)lds;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
    const uint8_t* qreq = (const uint8_t*)p.q + (size_t)b * p.rows * kRowBytes;
#pragma unroll
    for (int j = 0; j < 18; ++j) {
        const int qb = 18 * wv + j;
        const int q = qb * 64 + lane;
        const int r = q / kRowChunks;
        const int pc = q - r * kRowChunks;
        const uint32_t src = (uint32_t)min(mt * kMTile + r, p.rows - 1) * kRowBytes + ((pc ^ swz(r)) << 4);
        dma16(ring_addr + qb * 1024, qreq, src);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (A) {
        const lds_u8* qrow = ring + (s * 32 + lr) * kRowBytes;
        int qb4[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) qb4[k4] = (((2 * k4 + G) ^ swz(lr)) & 7) << 4;
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) qf[ks] = *(const lds_bf16x8*)(qrow + qb4[ks & 3] + (ks >> 2) * 128);
    }
    __syncthreads();   // the A waves hold their query fragments: the ring is free
}

// kRun: the piece may be a run of consecutive splits (Piece::run > 1).  The
// run streams through the ring as one sequence of half pages: where a split
// ends, wave A has already taken the next split's first half page through
// QK^T and the softmax (from a fresh max and sums), the copies of the next two
// are in flight, and the finished split leaves through the one ring slot that
// nothing uses then.
template <bool A, int kKAhead, bool kRun>
__device__ __forceinline__ void decode_bf16_ab_body(const DecodeParams& p, const Piece& w, uint8_t* lds,
                                                    const int s, const int wv, bf16x8_t (&qf)[36]) {
    const int lane = lane_id_fresh();
    const int tid = wv * 64 + lane;
    const int G = lane >> 5;        // MFMA k-group of this lane
    const int lr = lane & 31;       // query row (QK^T B operand, PV result) / token (QK^T A operand)
    const int b = w.b;
    const int n = min(max(p.seq_lens[b], 0), p.max_pages * kPage);
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    const uint8_t* kvbase = (const uint8_t*)p.kv;
    lds_u8* const ring = (lds_u8*)lds;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
    lds_u8* const pbase = (lds_u8*)lds + kAbPBufOff + lane * 16;   // + 8192 buf + 2048 tile + 1024 k-step

    const int half_begin = 2 * w.page_begin;
    const int half_end = min(2 * w.page_end, (n + kHalfTok - 1) / kHalfTok);
    auto slot_of = [&](int k) { return (k - half_begin) & 3; };
    auto slot_ptr = [&](int k) { return ring + slot_of(k) * kSlotBytes; };
    auto pfrag_ptr = [&](int k, int t, int k2) { return pbase + ((k - half_begin) & 1) * 8192 + t * 2048 + k2 * 1024; };

    // ---- page copies (B waves): a half page is 36 blocks of 1 KB (block j
    // holds LDS chunks 64 j .. 64 j + 63 = (token q / 72, position q % 72),
    // i.e. global chunk position ^ swz(token)); B wave of SIMD s copies the
    // blocks 9 s .. 9 s + 8.  Past the last half page a copy re-reads the
    // last one (a valid page whose data is never used), so that every step
    // issues the same copies.
    int cp_off[A ? 1 : 9];
    if (!A) {
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const int q = (9 * s + j) * 64 + lane;
            const int t = q / kRowChunks;
            const int pc = q - t * kRowChunks;
            cp_off[j] = t * kRowBytes + ((pc ^ swz(t)) << 4);
        }
    }
    const __attribute__((address_space(4))) int32_t* bt_s = (const __attribute__((address_space(4))) int32_t*)bt;
    auto page_id = [&](int k) { return clamp_page(bt_s[k >> 1], p.num_pages); };
    auto copy_src = [&](int k) { return k < half_end ? k : half_end - 1; };
    auto half_src_of = [&](int pid, int k) { return kvbase + (size_t)pid * kPageBytes + (k & 1) * kSlotBytes; };
    auto copy_half = [&](int k, int pid) {
        if (!A) {
            const uint8_t* src = half_src_of(pid, copy_src(k));
            const uint32_t dst = ring_addr + slot_of(k) * kSlotBytes + 9 * s * 1024;
#pragma unroll
            for (int j = 0; j < 9; ++j) dma16(dst + j * 1024, src, (uint32_t)cp_off[j]);
        }
    };

    // ---- this lane's query row (A) and the visible lengths
    const int row = w.mt * kMTile + s * 32 + lr;
    const bool row_ok = row < p.rows;
    const int tq = row / p.heads;
    const int unit_end = half_end * kHalfTok;
    const int nvis = min(p.causal ? max(n - (p.q_len - 1 - tq), 0) : n, unit_end);
    const int nvis_min = min(p.causal ? max(n - (p.q_len - 1), 0) : n, unit_end);


    // K fragment offsets within a slot (A): token lr, chunk 2 ks + G at position
    // (c & ~7) | ((c ^ swz(lr)) & 7); c(ks + 4) = c(ks) + 8, so four bases
    // cover the 36 k-steps with immediates 128 (ks / 4)
    int qk_off[A ? 4 : 1];
    if (A) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) qk_off[k4] = lr * kRowBytes + ((((2 * k4 + G) ^ swz(lr)) & 7) << 4);
    }
    // V^T transpose reads of dim tile dt = 4 s + j (chunk 4 dt + 2 (bk % 2) +
    // (lane % 4) / 2 of tokens 4 G + e and + 8): 16 s and 8 (j / 2) lie above
    // the 3 swizzled chunk bits, 4 (j % 2) inside them
    int tr_off[2];
    {
        const int li = lane & 15, e = li >> 2, cc = li & 3, dhl = (lane >> 4) & 1;
        const int t = 4 * G + e;
        const int sw = swz(t);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
            tr_off[d2] = t * kRowBytes + s * 256 + (((4 * d2 + 2 * dhl + (cc >> 1)) ^ sw) << 4) + (cc & 1) * 8;
    }
    auto vfrag = [&](lds_u8* cur, int j, int k2) -> bf16x8_t {
        const int off = tr_off[j & 1] + (j >> 1) * 128 + k2 * 16 * kRowBytes;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(cur + off));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(cur + ((off ^ 32) + 8 * kRowBytes)));
        return __builtin_bit_cast(bf16x8_t, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    // O^T accumulators for the rows of tile t over dim tile 4 s + J0 + j (A:
    // j = 0; B: j = 0 .. 2): oa[t] (j = 0) and ov[j - 1][t], all in VGPRs;
    // element i is dim + 8 (i / 4) + 4 G + i % 4
    constexpr int NJ = A ? 1 : 3;
    constexpr int J0 = A ? 0 : 1;
    f32x16 oa[4], ov[A ? 1 : 2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        oa[t] = (f32x16)0.f;
        asm volatile("" : "+v"(oa[t]));
    }
    if (!A) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ov[j][t] = (f32x16)0.f;
                asm volatile("" : "+v"(ov[j][t]));
            }
    }
    // O^T[j][t] += V^T . P^T (inline assembly with the accumulator tied to its
    // registers, so the compiler never moves it)
    auto mfma_o = [&](int j, int t, const bf16x8_t& a, const bf16x8_t& bp) {
        if (j == 0) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(oa[t]) : "v"(a), "v"(bp));
        else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(ov[j - 1][t]) : "v"(a), "v"(bp));
    };
    auto o_elem = [&](int j, int t, int i) -> float { return j == 0 ? oa[t][i] : ov[j - 1][t][i]; };
    // (A) reference max (whole log2 units) and this lane's shares of the row
    // sum: l of the weights as computed (for the LSE) and lr of the weights as
    // rounded to bf16, the values the PV multiplies (for normalising O, so that
    // the output is a weighted mean of V whatever the rounding)
    float m = -INFINITY, l = 0.f, lr_sum = 0.f;
    auto pv_drain = [&]() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); };
    // o *= a for the accumulators of row tile t, in place
    auto scale_tile = [&](int t, float a) {
        oa[t] *= a;
        if (!A) {
#pragma unroll
            for (int j = 0; j < 2; ++j) ov[j][t] *= a;
        }
    };

    // O^T += V^T . P^T over half page k for this wave's dim tiles and the four
    // row tiles.  The four k-step 0 P fragments are read first (with A's first
    // V fragment): their first words hold the flag bits, so one LDS round trip
    // serves the check and the first MFMAs; every wave reads the same bits, so
    // when a row of some tile moved its reference max (rare) the whole
    // workgroup takes the slow path together: each wave rescales its
    // accumulators of the tile by 2^-d, and after a barrier the tile's A wave
    // clears the sign bits in LDS (a second barrier publishes them; the
    // fragments are then read again) before the usual PV.
    auto pv = [&](int k) {
        lds_u8* cur = slot_ptr(k);
        int flag = 0;
        bf16x8_t a0, pt0[4];
        if (A) a0 = vfrag(cur, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            pt0[t] = *(const lds_bf16x8*)pfrag_ptr(k, t, 0);
            flag |= __builtin_bit_cast(i32x4, pt0[t])[0];
        }
        if (__builtin_expect(__any((flag & 0x8000) != 0), 0)) {
            pv_drain();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const i32x4 v = *(const __attribute__((address_space(3))) i32x4*)pfrag_ptr(k, t, 0);
                int d = ((unsigned)v[0]) >> 31;
#pragma unroll
                for (int q = 1; q < 4; ++q)
                    d |= (((v[q] >> 15) & 1) << (2 * q - 1)) | ((((unsigned)v[q]) >> 31) << (2 * q));
                if (!((v[0] >> 15) & 1)) d = 0;
                if (__any(d != 0)) scale_tile(t, __builtin_ldexpf(1.f, -d));
            }
            __syncthreads();
            if (A) {
                __attribute__((address_space(3))) i32x4* f = (__attribute__((address_space(3))) i32x4*)pfrag_ptr(k, s, 0);
                i32x4 v = *f;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] &= 0x7fff7fff;
                *f = v;
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 4; ++t) pt0[t] = *(const lds_bf16x8*)pfrag_ptr(k, t, 0);
        }
        if (A) {
            // one dim tile: each V fragment feeds four MFMAs, the four P
            // fragments of a k-step read at once
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const bf16x8_t a = k2 == 0 ? a0 : vfrag(cur, 0, k2);
                bf16x8_t pt[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) pt[t] = k2 == 0 ? pt0[t] : *(const lds_bf16x8*)pfrag_ptr(k, t, k2);
#pragma unroll
                for (int t = 0; t < 4; ++t) mfma_o(0, t, a, pt[t]);
            }
        } else {
            // three dim tiles: the four P fragments of a k-step stay in
            // registers, each V fragment (read one ahead) feeds four MFMAs
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                bf16x8_t pt[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) pt[t] = k2 == 0 ? pt0[t] : *(const lds_bf16x8*)pfrag_ptr(k, t, k2);
                bf16x8_t vc = vfrag(cur, J0, k2);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    bf16x8_t vn;
                    if (j + 1 < NJ) vn = vfrag(cur, J0 + j + 1, k2);
#pragma unroll
                    for (int t = 0; t < 4; ++t) mfma_o(j, t, vc, pt[t]);
                    vc = vn;
                }
            }
        }
    };

    // (A) S^T of half page k for the wave's 32 rows: all 36 k-steps in one
    // accumulation chain, K fragments read kKAhead ahead (inline-assembly MFMAs
    // with S tied to VGPRs; the 12 wait states an 8-pass MFMA's result needs
    // before a VALU instruction reads or writes it follow the chain)
    auto qk = [&](int k, f32x16& sacc) {
        lds_u8* cur = slot_ptr(k);
        bf16x8_t kf[kKAhead];
#pragma unroll
        for (int ks = 0; ks < kKAhead; ++ks) kf[ks] = *(const lds_bf16x8*)(cur + qk_off[ks & 3] + (ks >> 2) * 128);
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
            const bf16x8_t a = kf[ks % kKAhead];
            if (ks + kKAhead < 36)
                kf[ks % kKAhead] = *(const lds_bf16x8*)(cur + qk_off[(ks + kKAhead) & 3] + ((ks + kKAhead) >> 2) * 128);
            if (ks == 0)
                asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(a), "v"(qf[ks]));
            else
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(a), "v"(qf[ks]));
        }
        asm volatile("s_nop 7\n\ts_nop 3" : "+v"(sacc));
    };
    // (A) online softmax of half page k: masks invisible tokens (element i is
    // token 32 k + 8 (i / 4) + 4 G + i % 4), moves the reference max (whole
    // log2 units) when the row max exceeds it by more than kRescaleSlackAb,
    // and publishes both k-step fragments of P^T; the k-step 0 fragment
    // carries the shift d when some row of the tile moved
    const float c_log2 = p.scale_log2;
    auto softmax = [&](int k, f32x16& sacc) {
        if (k * kHalfTok + kHalfTok > nvis_min) {
            const int lim = nvis - k * kHalfTok - 4 * G;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = (8 * (i >> 2) + (i & 3)) < lim ? sacc[i] : -INFINITY;
        }
        // (a v_max3 tree: fmaxf would first quiet every MFMA result)
        const float q0 = max3f(sacc[0], sacc[1], sacc[2]), q1 = max3f(sacc[3], sacc[4], sacc[5]),
                    q2 = max3f(sacc[6], sacc[7], sacc[8]), q3 = max3f(sacc[9], sacc[10], sacc[11]),
                    q4 = max3f(sacc[12], sacc[13], sacc[14]);
        float mx = max3f(max3f(q0, q1, q2), max3f(q3, q4, sacc[15]), q0);
        mx = pair_max(mx) * c_log2;
        const bool grow = mx > m + kRescaleSlackAb;
        const float m_new = grow ? __builtin_ceilf(mx) : m;
        // (nothing has been accumulated while m is still -inf: no rescale)
        const int d = grow && m != -INFINITY ? (int)fminf(m_new - m, 127.f) : 0;
        m = m_new;
        l *= __builtin_ldexpf(1.f, -d);
        lr_sum *= __builtin_ldexpf(1.f, -d);
        const float mneg = m == -INFINITY ? 0.f : -m;
        float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sacc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c_log2, mneg));
            if (i & 1) sum1 += sacc[i]; else sum0 += sacc[i];
        }
        l += sum0 + sum1;
        bf16x8_t pf0, pf1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pf0[e] = (__bf16)sacc[e];
            pf1[e] = (__bf16)sacc[8 + e];
        }
        i32x4 v = __builtin_bit_cast(i32x4, pf0);
        {
            const i32x4 v1 = __builtin_bit_cast(i32x4, pf1);
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r0 += __int_as_float(v[q] << 16) + __int_as_float(v[q] & (int)0xffff0000u);
                r1 += __int_as_float(v1[q] << 16) + __int_as_float(v1[q] & (int)0xffff0000u);
            }
            lr_sum += r0 + r1;
        }
        if (__builtin_expect(__any(d != 0), 0)) {
            const int f = d != 0 ? 1 : 0;
            v[0] |= (f << 15) | ((d & 1) << 31);
#pragma unroll
            for (int q = 1; q < 4; ++q) v[q] |= (((d >> (2 * q - 1)) & 1) << 15) | (((d >> (2 * q)) & 1) << 31);
        }
        *(__attribute__((address_space(3))) i32x4*)pfrag_ptr(k, s, 0) = v;
        *(lds_bf16x8*)pfrag_ptr(k, s, 1) = pf1;
    };
    // (B) zero the rows of half page k past the sequence end (they may hold
    // anything, NaN included), so that a zero weight times V stays zero; runs
    // after the copies of k have landed, and the next barrier orders it before
    // any PV of k (a concurrent QK^T of k only reads masked tokens there)
    auto zero_tail = [&](int k) {
        const int t0 = n - k * kHalfTok;
        if (t0 >= kHalfTok) return;
        lds_u8* cur = slot_ptr(k);
        const int tid = s * 64 + lane;
        for (int idx = tid; idx < (kHalfTok - t0) * kRowChunks; idx += 256) {
            const int t = t0 + idx / kRowChunks;
            const int c = idx % kRowChunks;
            *(__attribute__((address_space(3))) i32x4*)(cur + t * kRowBytes + c * 16) = (i32x4)0;
        }
    };

    // (run) the split of half page k is (k - half_begin) / (2 run_pages); its
    // partial goes to slot w.slot + j m_tiles
    const int run = kRun ? w.run : 1;
    int j_cur = 0;
    auto split_slot = [&](int j) { return w.slot + j * p.plan.m_tiles; };

    // ---- a split's end: o = O / l for this wave's dim tiles of the four row
    //      tiles; lse = ln(sum exp) for the A wave's rows
    auto zero_o = [&]() {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            oa[t] = (f32x16)0.f;
            asm volatile("" : "+v"(oa[t]));
        }
        if (!A) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    ov[j][t] = (f32x16)0.f;
                    asm volatile("" : "+v"(ov[j][t]));
                }
        }
    };
    auto write_lse = [&](int slot_j, float m_f, float l_row) {
        if (A && row_ok && G == 0) {
            const float lse = l_row > 0.f ? (m_f + __log2f(l_row)) * kLn2 : -INFINITY;
            if (w.nsplit == 1) p.lse[(size_t)b * p.rows + row] = lse;
            else p.ws_lse[(size_t)slot_j * kMTile + (row - w.mt * kMTile)] = lse;
        }
    };
    // Inside a run, where split j ends after half page k (m_f, l_f, lr_f: its
    // max and this lane's sums): the copies of half pages k + 2 and k + 3 are
    // in flight and k + 1 holds the next split's first weights, so the rows
    // leave 32 at a time (one row tile) through half page k's slot, as bf16
    // partials (rows of 1,040 bytes; the rounded weights' sums after the 32
    // rows).  B first waits for the copy of k + 2, so that its stores never
    // stand between a wait and the copy it waits for.
    auto finish_mid = [&](int k, int slot_j, float m_f, float l_f, float lr_f) {
        if (!A) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
        pv_drain();
        const float l_row = pair_sum(l_f);
        const float lr_row = pair_sum(lr_f);
        // (every lane-dependent address here comes from a fresh lane id: the
        // compiler would otherwise keep them in registers across the loop)
        const int lf = lane_id_fresh();
        const int lrf = lf & 31, Gf = lf >> 5;
        constexpr int st_row = kV * 2 + 16;
        constexpr int row_chunks = kV * 2 / 16;
        static_assert(32 * st_row + 4 * 32 * 4 <= kSlotBytes, "one row tile and the sums fit a ring slot");
        lds_u8* const stage = slot_ptr(k);
        lds_f32* const lb = (lds_f32*)(stage + 32 * st_row);
        __syncthreads();                  // every wave is done with half page k
        if (A && Gf == 0) lb[s * 32 + lrf] = lr_row;
        __syncthreads();
        float lt[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) lt[t] = lb[t * 32 + lrf];
        // the lse before the rows: any load after the stores (an address
        // reloaded from scratch, say) would wait for them
        if (A && Gf == 0 && w.mt * kMTile + s * 32 + lrf < p.rows)
            p.ws_lse[(size_t)slot_j * kMTile + s * 32 + lrf] = l_row > 0.f ? (m_f + __log2f(l_row)) * kLn2 : -INFINITY;
        uint8_t* const gbase = (uint8_t*)p.ws_o + (size_t)slot_j * kMTile * kV * 2;
        lds_u8* const srow0 = stage + lrf * st_row + 2 * (32 * (4 * s + J0) + 4 * Gf);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float inv = lt[t] > 0.f ? 1.f / lt[t] : 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 v = (f32x4){o_elem(j, t, 4 * q4), o_elem(j, t, 4 * q4 + 1), o_elem(j, t, 4 * q4 + 2),
                                            o_elem(j, t, 4 * q4 + 3)} * inv;
                    __bf16 __attribute__((ext_vector_type(4))) h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) h[i] = (__bf16)v[i];
                    *(lds_i16x4*)(srow0 + 2 * 32 * j + 2 * 8 * q4) = __builtin_bit_cast(i16x4, h);
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = wv * 64 + lf; i < 32 * row_chunks; i += 512) {
                const int rl = i / row_chunks, c = i - rl * row_chunks;
                if (w.mt * kMTile + 32 * t + rl < p.rows)
                    *(i32x4*)(gbase + (size_t)(32 * t + rl) * kV * 2 + 16 * c) =
                        *(const __attribute__((address_space(3))) i32x4*)(stage + rl * st_row + 16 * c);
            }
            __syncthreads();
        }
        zero_o();
    };

    if (half_begin < half_end) {
        // prologue: B copies the first three half pages; T(pre): the first has
        // landed; A contracts it and publishes P of the first half page
        int pid_next = 0;
        if (!A) {
            const int pid0 = page_id(half_begin);
            const int pid1 = page_id(copy_src(half_begin + 1));
            const int pid2 = page_id(copy_src(half_begin + 2));
            copy_half(half_begin, pid0);
            copy_half(half_begin + 1, pid1);
            copy_half(half_begin + 2, pid2);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));
            pid_next = page_id(copy_src(half_begin + 3));
        }
        lds_sync();
        // (the first half page's tail is zeroed before the next barrier, and
        // its PV runs after it)
        if (!A) zero_tail(half_begin);
        if (A) {
            f32x16 sacc;
            qk(half_begin, sacc);
            softmax(half_begin, sacc);
        }
        // (run) the first half page of the next split, and whether the last
        // step ended a split (its end already waited for the copy that this
        // step's barrier would wait for)
        int next_split = kRun && run > 1 ? half_begin + 2 * w.run_pages : half_end;
        bool after_split = false;
        for (int k = half_begin;; ++k) {
            // T(k): the copies of half page k + 1 have landed (B waits for its
            // own, the barrier makes them everyone's), P(k) is published
            if (!A && !(kRun && after_split)) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
            lds_sync();
            const bool more = k + 1 < half_end;
            const bool ends = kRun && more && k + 1 == next_split;
            float m_f = 0.f, l_f = 0.f, lr_f = 0.f;
            if (A) {
                pv(k);
                if (more) {
                    f32x16 sacc;
                    qk(k + 1, sacc);
                    if (ends) {
                        // half page k + 1 opens the next split: its softmax
                        // starts from no max and empty sums
                        m_f = m; l_f = l; lr_f = lr_sum;
                        m = -INFINITY; l = 0.f; lr_sum = 0.f;
                    }
                    softmax(k + 1, sacc);
                }
            } else {
                copy_half(k + 3, pid_next);
                pid_next = page_id(copy_src(k + 4));
                if (more) zero_tail(k + 1);
                pv(k);
            }
            if (kRun) {
                after_split = ends;
                if (ends) {
                    finish_mid(k, split_slot(j_cur), m_f, l_f, lr_f);
                    ++j_cur;
                    next_split += 2 * w.run_pages;
                }
            }
            if (!more) break;
        }
    }

    // ---- the last split's end (the whole ring is free): rows leave through the
    // ring, per half (64 rows): every wave writes its dims of the rows, scaled
    // by 1 / l, as fp32 (a single piece to an fp32 output) or bf16 (a bf16
    // output, or a split partial), into rows of 512 e + 16 bytes; then the
    // workgroup stores whole contiguous row pieces, 16 bytes per lane.
    auto finish = [&](int slot_j) {
        // No copy may still be writing this workgroup's LDS when it is reused.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        pv_drain();
        const float l_row = pair_sum(l);
        const float lr_row = pair_sum(lr_sum);
        __syncthreads();                      // every wave is done with the ring and the P buffers
        lds_f32* const lbuf = (lds_f32*)(lds + kAbPBufOff);   // [4 tiles][32 rows]: sums of the rounded weights
        if (A && G == 0) lbuf[s * 32 + lr] = lr_row;
        __syncthreads();
        float lt[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) lt[t] = lbuf[t * 32 + lr];
        const bool f32 = w.nsplit == 1 && !p.out_bf16;
        const int e = f32 ? 4 : 2;
        const int st_row = kV * e + 16;
        const int row_chunks = kV * e / 16;
        uint8_t* gbase = w.nsplit > 1 ? (uint8_t*)p.ws_o + (size_t)slot_j * kMTile * kV * 2
                                      : (uint8_t*)p.out + ((size_t)b * p.rows + (size_t)w.mt * kMTile) * kV * e;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int t = 2 * hf + tt;
                const float inv = lt[t] > 0.f ? 1.f / lt[t] : 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    lds_u8* srow = ring + (32 * tt + lr) * st_row + e * (32 * (4 * s + J0 + j) + 4 * G);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 v = (f32x4){o_elem(j, t, 4 * q4), o_elem(j, t, 4 * q4 + 1), o_elem(j, t, 4 * q4 + 2),
                                                o_elem(j, t, 4 * q4 + 3)} * inv;
                        if (f32) {
                            *(__attribute__((address_space(3))) f32x4*)(srow + 4 * 8 * q4) = v;
                        } else {
                            __bf16 __attribute__((ext_vector_type(4))) h;
#pragma unroll
                            for (int i = 0; i < 4; ++i) h[i] = (__bf16)v[i];
                            *(lds_i16x4*)(srow + 2 * 8 * q4) = __builtin_bit_cast(i16x4, h);
                        }
                    }
                }
            }
            __syncthreads();
            for (int i = (int)tid; i < 64 * row_chunks; i += 512) {
                const int rl = i / row_chunks, c = i - rl * row_chunks;
                if (w.mt * kMTile + 64 * hf + rl < p.rows)
                    *(i32x4*)(gbase + (size_t)(64 * hf + rl) * kV * e + 16 * c) =
                        *(const __attribute__((address_space(3))) i32x4*)(ring + rl * st_row + 16 * c);
            }
            __syncthreads();
        }
        write_lse(slot_j, m, l_row);
    };
    finish(split_slot(j_cur));
    if (kRun) {
        // splits of the run past the sequence's end: empty partials (zero
        // rows, lse -inf)
        for (int j = j_cur + 1; j < run; ++j) {
            zero_o();
            m = -INFINITY; l = 0.f; lr_sum = 0.f;
            finish(split_slot(j));
        }
    }
}

// kGroups: the instance for work lists that may hold groups of splits (a
// group runs as one stream of half pages, K fragments one ahead: with two
// ahead the split ends inside the loop would not fit the registers); the
// other instance runs single-piece items only.
template <bool kGroups>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_bf16_ab_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kAbLdsBytes];
    const WorkItem w = decode_work_item<512>(p, lds);
    if (w.b < 0) return;
    // roles: each wave posts its SIMD; with two waves on every SIMD the lower
    // wave index of a SIMD is A and the SIMD id names the row tile and dim
    // tiles; otherwise waves 0-3 are A (tile = wave) and 4-7 B
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sid = __builtin_amdgcn_readfirstlane(hw_simd_id());
    lds_int* tab = (lds_int*)lds;
    if ((threadIdx.x & 63) == 0) tab[wv] = sid;
    __syncthreads();
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, cnt3 = 0, lower = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int si = __builtin_amdgcn_readfirstlane(tab[i]);
        cnt0 += si == 0; cnt1 += si == 1; cnt2 += si == 2; cnt3 += si == 3;
        lower += (si == sid && i < wv) ? 1 : 0;
    }
    __syncthreads();   // the table's LDS is reused for the query
    const bool by_hw = cnt0 == 2 && cnt1 == 2 && cnt2 == 2 && cnt3 == 2;
    const bool is_a = by_hw ? lower == 0 : wv < 4;
    const int s = by_hw ? sid : (wv & 3);
    bf16x8_t qf[36];
    if constexpr (kGroups) {
        const Piece pc = group_piece(p, w);
        if (pc.nsplit > 1 && (pc.run < 1 || pc.slot >= p.plan.units_max)) return;   // (a stored item past the partial slots)
        if (is_a) {
            stage_query_bf16<true>(p, pc.b, pc.mt, lds, s, wv, qf);
            decode_bf16_ab_body<true, 1, true>(p, pc, lds, s, wv, qf);
        } else {
            stage_query_bf16<false>(p, pc.b, pc.mt, lds, s, wv, qf);
            decode_bf16_ab_body<false, 1, true>(p, pc, lds, s, wv, qf);
        }
    } else {
        // (an item holding a group is not followed here: the plan for this
        // instance makes none, see PlanParams::group_ok)
        if (w.chunk <= 0 && w.g0 > 1) return;
        const Piece pc = single_piece(p, w);
        if (pc.nsplit > 1 && (pc.slot < 0 || pc.slot >= p.plan.units_max)) return;
        if (is_a) {
            stage_query_bf16<true>(p, pc.b, pc.mt, lds, s, wv, qf);
            decode_bf16_ab_body<true, 2, false>(p, pc, lds, s, wv, qf);
        } else {
            stage_query_bf16<false>(p, pc.b, pc.mt, lds, s, wv, qf);
            decode_bf16_ab_body<false, 2, false>(p, pc, lds, s, wv, qf);
        }
    }
}

// ---------------------------------------------------------------------------
// split-KV decode, OCP fp8 e4m3 cache and query: shared layout and helpers
//
// The work items, the ring of 4 LDS slots and the direct HBM -> LDS loads
// are the bf16 kernel's, with these differences:
//  - one ring slot holds a whole 64-token page (64 x 576 bytes = 36,864);
//  - both contractions run on v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8 ->
//    fp32, K = 64 per instruction):
//      S^T[32 tok][32 rows]  += K[32 tok][64 dims] . Q^T[64 dims][32 rows]
//      O^T[32 dims][32 rows] += V^T[32 dims][64 tok] . P^T[64 tok][32 rows]
//    so a page is 2 token tiles x 9 k-steps of QK^T and one PV MFMA per
//    32-dim tile and row tile;
//  - the weights enter the PV product as two e4m3 terms, hi = e4m3(w) and
//    lo = e4m3(w - hi), one MFMA each, so that their error is about 2^-8 of
//    w instead of the 2^-4 of a single e4m3 rounding (which alone exceeds a
//    few 1e-2 on short, peaked rows).  Weights are offset by 2^3 so that they
//    span (0, 2^8]; the reference max takes integer values (log2 units) and
//    moves once the row max exceeds it by 5, so every rescale factor is an
//    exact power of two 2^-d; d (8 bits) rides in the sign bits of hi bytes
//    0-7, which are free because the weights are non-negative;
//  - the per-tensor cache scale multiplies the logits (folded into the exp2
//    factor) and the output (in the epilogue); the query scale arrives folded
//    into `scale`.
// Operand layouts of the 32x32x64 fp8 MFMA: lane L supplies row (A) or
// column (B) L % 32 and 32 consecutive k values 32 (L / 32) .. + 31 of it,
// one byte each; the result layout is the one of every 32x32 f32 MFMA.
//
// LDS row layout: token t of the page occupies 576 bytes = 36 chunks of 16;
// chunk c sits at position c ^ swz8(t), swz8(t) = (t / 4) % 4 (a permutation
// inside aligned groups of 4 chunks), which puts 16 consecutive tokens, and
// the 8 tokens of a V^T transpose read, on distinct banks.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kRowBytes8 = kQK;                    // 576 bytes per fp8 cache row
constexpr int kPageBytes8 = kPage * kRowBytes8;    // 36,864 = one ring slot
constexpr int kRowChunks8 = kRowBytes8 / 16;       // 36
constexpr float kRescaleSlack8 = 5.f;              // reference max moves when the max grows by > 2^5
constexpr float kWeightOffset8 = 3.f;              // weights are exp2(s c - m + 3) <= 2^8 < 448
static_assert(kPageBytes8 == kSlotBytes, "an fp8 page fills exactly one ring slot");

// d (0..255) into the sign bits of the bytes of two dwords (bits 8 i + 7),
// and back: each is a multiply that spreads / gathers one nibble without carries.
__device__ __forceinline__ int spread_nibble(int x) { return (int)(((uint32_t)(x & 15) * 0x10204080u) & 0x80808080u); }
__device__ __forceinline__ int gather_nibble(int w) {
    return (int)(((((uint32_t)w >> 7) & 0x01010101u) * 0x01020408u) >> 24) & 15;
}

__device__ __forceinline__ int swz8(int t) { return (t >> 2) & 3; }


__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
    return (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Four e4m3 codes (round to nearest even, saturating) of v[0..3] in one dword.
// (old: any value; both halves of it are replaced.  Passing the register the
// result will overwrite saves the zero a constant would be moved in with.)
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d, int old = 0) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// ---------------------------------------------------------------------------
// split-KV decode, fp8 cache, two waves per SIMD with split roles
//
// Workgroup = 8 waves (two per SIMD) over one work item of kMTile = 128 query
// rows.  The softmax's VALU work (two e4m3 weight terms per logit) would take
// turns with the MFMAs on a single wave; the two waves of a SIMD split the
// work of one 32-row tile (rows 32 s .. 32 s +
// 31 on SIMD s):
//  - wave A holds the tile's Q^T (9 k-steps, 72 VGPRs), contracts QK^T over the
//    page (2 token tiles x 9 k-steps), runs the online softmax (reference max
//    in whole log2 units, moved when the row max exceeds it by 5), forms the
//    hi and lo e4m3 weight terms, and accumulates O^T for dim tiles 0 .. 2
//    (96 dims, 48 VGPRs);
//  - wave B accumulates O^T for dim tiles 3 .. 15 (416 dims, 208 VGPRs) and
//    issues the page copies.
// Each V^T fragment read from LDS feeds two MFMAs (hi and lo term).  Every
// SIMD reads all of V (its own row tile) but only its own tile's weights: P^T
// goes from A to B of the same SIMD, never across SIMDs.
//
// LDS: the 4-slot ring of pages (147,456 bytes) and one P^T buffer per tile
// (hi 2 KB + lo 2 KB, 16 KB): the whole 160 KB, so P^T is single-buffered and
// each page step has two barriers:
//   T(k): page k + 1 has landed, P(k) is published, every wave is past its
//         reads of page k - 1 (B refills that slot with page k + 3);
//   M(k): B holds P(k) in registers, so A may overwrite it with P(k + 1).
// Phase 1 (T(k) .. M(k)): A contracts QK^T of page k + 1 (18 MFMAs); B reads
// P(k) (the rescale shift d rides in the sign bits of hi bytes 0 - 7, as
// described above), issues the copy of page k + 3 and zeroes a sequence tail.
// Phase 2 (M(k) .. T(k + 1)): A runs the softmax of page k + 1, with its PV
// share of page k (6 MFMAs, the weights of page k still in its registers)
// issued between the softmax's pieces, and publishes P(k + 1); B runs the PV
// of page k (26 MFMAs), so A's VALU work overlaps the MFMAs.
// Roles follow the hardware SIMD of each wave (as in the bf16 two-role kernel).
// ---------------------------------------------------------------------------
constexpr int kAb8PBufOff = kRingBytes;                 // [tile][hi, lo][half][lane] 16 B
constexpr int kAb8LdsBytes = kAb8PBufOff + 4 * 4096;    // 163,840 (the whole LDS)
static_assert(kAb8LdsBytes <= 163840, "LDS budget");
constexpr int kAb8DimTilesA = 3;                        // O^T dim tiles of wave A (B: the other 13)
constexpr int kAb8KAhead = 2;                           // K fragment pairs in flight during QK^T

template <bool A>
__device__ __forceinline__ void decode_fp8_ab_body(const DecodeParams& p, const Piece& w, uint8_t* lds,
                                                   const int s, const int wv) {
    const int lane = lane_id_fresh();
    const int G = lane >> 5;        // MFMA k-half of this lane (0/1)
    const int lr = lane & 31;       // query row (QK B operand, PV result) / token (QK A operand)
    const int b = w.b;
    const int n = min(max(p.seq_lens[b], 0), p.max_pages * kPage);
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    const uint8_t* kvbase = (const uint8_t*)p.kv;
    lds_u8* const ring = (lds_u8*)lds;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
    // this tile's P^T buffer: hi at + 0, lo at + 2048, k-half tiles 1024 apart
    lds_u8* const pbuf = (lds_u8*)lds + kAb8PBufOff + s * 4096 + lane * 16;
    const float kv_scale = *p.kv_scale;
    const float c_exp = p.scale_log2 * kv_scale;   // logits in log2 units per unit of q.k

    const int pg_begin = w.page_begin;
    const int pg_end = min(w.page_end, (n + kPage - 1) / kPage);
    auto slot_ptr = [&](int k) { return ring + ((k - pg_begin) & 3) * kSlotBytes; };

    // ---- page copies (B): B wave of SIMD s copies tokens 16 s .. 16 s + 15 of
    // a page (9 blocks of 1 KB, LDS chunk q = 64 j + lane of the block holds
    // token q / 36, position q % 36 = global chunk position ^ swz8(token)).
    // Past the last page a copy re-reads the last one (a valid page whose data
    // is never used), so that every step issues the same copies.
    // (offsets recomputed per copy: B has no registers to keep nine of them)
    auto cp_off = [&](int j) {
        const int qc = j * 64 + lane_id_fresh();
        const int t = qc / kRowChunks8;
        const int pc = qc - t * kRowChunks8;
        return t * kRowBytes8 + ((pc ^ swz8(t)) << 4);
    };
    const __attribute__((address_space(4))) int32_t* bt_s = (const __attribute__((address_space(4))) int32_t*)bt;
    auto page_id = [&](int k) { return clamp_page(bt_s[k], p.num_pages); };
    auto copy_src = [&](int k) { return k < pg_end ? k : pg_end - 1; };
    auto copy_page = [&](int k, int pid) {
        if (!A) {
            const uint8_t* src = kvbase + (size_t)pid * kPageBytes8 + s * 16 * kRowBytes8;
            const uint32_t dst = ring_addr + ((k - pg_begin) & 3) * kSlotBytes + s * 9 * 1024;
#pragma unroll
            for (int j = 0; j < 9; ++j) dma16(dst + j * 1024, src, (uint32_t)cp_off(j));
        }
    };

    const int row = w.mt * kMTile + s * 32 + lr;
    const bool row_ok = row < p.rows;
    const int tq = row / p.heads;
    const int unit_end = pg_end * kPage;
    const int nvis = min(p.causal ? max(n - (p.q_len - 1 - tq), 0) : n, unit_end);
    const int nvis_min = min(p.causal ? max(n - (p.q_len - 1), 0) : n, unit_end);

    // PV A operands (V^T, 32 dims x 64 tokens) by transpose reads: dim tile
    // D reads at tr_off[D % 2] + 64 (D / 2) (the
    // swizzle permutes chunks inside aligned groups of 4, and 2 D + (lane / 16) % 2
    // stays in the group of chunk 4 (D / 2))
    int tr_off[2];
    {
        const int gl = lane >> 4, sl = lane & 15, kh = gl >> 1;
        const int t0 = 4 * kh + 8 * (sl >> 3) + ((sl >> 1) & 3);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
            const int c = 2 * d2 + (gl & 1);
            tr_off[d2] = t0 * kRowBytes8 + ((c ^ swz8(t0)) << 4) + 8 * (sl & 1);
        }
    }
    auto vfrag = [&](lds_u8* cur, int D) -> i32x8 {
        const int off = tr_off[D & 1] + (D >> 1) * 64;
        const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(cur + off));
        const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(cur + off + 16 * kRowBytes8));
        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(cur + off + 32 * kRowBytes8));
        const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(cur + off + 48 * kRowBytes8));
        return (i32x8){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    };

    // O^T accumulators of this wave's dim tiles (element i: dim 32 D + 8 (i / 4)
    // + 4 G + i % 4 of row lr), in VGPRs
    constexpr int ND = A ? kAb8DimTilesA : 16 - kAb8DimTilesA;
    constexpr int D0 = A ? 0 : kAb8DimTilesA;
    f32x16 o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) {
        o[j] = (f32x16)0.f;
        asm volatile("" : "+v"(o[j]));
    }
    auto mfma_o = [&](int j, const i32x8& a, const i32x8& bp) {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(o[j]) : "v"(a), "v"(bp));
    };

    auto pv_drain = [&]() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); };
    // o *= f, then the wait states a VALU write needs before an MFMA reads
    // the register (the rescale sits in a branch, where the build's wait-state
    // check does not look, and the next MFMA accumulates into o[0])
    auto scale_o = [&](float f) {
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            o[j] *= f;
            asm volatile("" : "+v"(o[j]));
        }
        asm volatile("s_nop 4");
    };
    // (A) reference max (whole log2 units) and this lane's share of the row sum
    float m = -INFINITY, l = 0.f;

    // (B) zero the rows of page k past the sequence end (they may hold
    // anything, NaN included), so that a zero weight times V stays zero; runs
    // once page k has landed, and a barrier orders it before any PV of k (a
    // concurrent QK^T of k only reads masked tokens there)
    auto zero_tail = [&](int k) {
        const int t0 = n - k * kPage;     // callers pass pages holding >= 1 token
        if (t0 >= kPage) return;
        lds_u8* cur = slot_ptr(k);
        for (int idx = s * 64 + lane; idx < (kPage - t0) * kRowChunks8; idx += 256) {
            const int t = t0 + idx / kRowChunks8;
            const int c = idx % kRowChunks8;
            *(lds_i32x4*)(cur + t * kRowBytes8 + c * 16) = (i32x4)0;
        }
    };

    if constexpr (A) {
        // Q^T fragments: k-step ks covers dims 64 ks .. + 63; lane holds dims 64 ks + 32 G .. + 31
        i32x8 qf[9];
        {
            const uint8_t* qr = (const uint8_t*)p.q + ((size_t)b * p.rows + min(row, p.rows - 1)) * kQK + 32 * G;
#pragma unroll
            for (int ks = 0; ks < 9; ++ks) {
                const i32x4 lo = *(const i32x4*)(qr + 64 * ks);
                const i32x4 hi = *(const i32x4*)(qr + 64 * ks + 16);
                qf[ks] = cat8(lo, hi);
            }
        }
        // QK A fragments: token 32 tau + lr, chunks 4 ks + 2 G + e at positions
        // 4 ks + ((2 G + e) ^ swz8(lr))
        int qk_off[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) qk_off[e] = lr * kRowBytes8 + (((2 * G + e) ^ swz8(lr)) << 4);
        auto kfrag = [&](lds_u8* cur, int tau, int ks) -> i32x8 {
            const i32x4 lo = *(const lds_i32x4*)(cur + qk_off[0] + tau * 32 * kRowBytes8 + 64 * ks);
            const i32x4 hi = *(const lds_i32x4*)(cur + qk_off[1] + tau * 32 * kRowBytes8 + 64 * ks);
            return cat8(lo, hi);
        };
        // S^T of page k: two token tiles, 9 k-steps each, as two interleaved
        // accumulation chains; K fragments read kAb8KAhead k-steps ahead;
        // between(ks) runs after MFMA pair ks
        auto qk = [&](int k, f32x16& s0, f32x16& s1, auto&& between) {
            lds_u8* cur = slot_ptr(k);
            constexpr int KA = kAb8KAhead;
            i32x8 kf0[KA], kf1[KA];
#pragma unroll
            for (int ks = 0; ks < KA; ++ks) {
                kf0[ks] = kfrag(cur, 0, ks);
                kf1[ks] = kfrag(cur, 1, ks);
            }
#pragma unroll
            for (int ks = 0; ks < 9; ++ks) {
                const i32x8 a0 = kf0[ks % KA], a1 = kf1[ks % KA];
                if (ks + KA < 9) {
                    kf0[ks % KA] = kfrag(cur, 0, ks + KA);
                    kf1[ks % KA] = kfrag(cur, 1, ks + KA);
                }
                if (ks == 0) {
                    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0"
                                 : "=&v"(s0) : "v"(a0), "v"(qf[ks]));
                    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0"
                                 : "=&v"(s1) : "v"(a1), "v"(qf[ks]));
                } else {
                    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0"
                                 : "+v"(s0) : "v"(a0), "v"(qf[ks]));
                    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0"
                                 : "+v"(s1) : "v"(a1), "v"(qf[ks]));
                }
                between(ks);
            }
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
        };
        // element i of token tile tau is token 64 k + 32 tau + 8 (i / 4) + 4 G + i % 4
        auto mask_s = [&](int k, f32x16& s0, f32x16& s1) {
            const int lim = nvis - k * kPage - 4 * G;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 8 * (i >> 2) + (i & 3);
                s0[i] = t < lim ? s0[i] : -INFINITY;
                s1[i] = t + 32 < lim ? s1[i] : -INFINITY;
            }
        };
        auto needs_mask = [&](int k) { return k * kPage + kPage > nvis_min; };

        // Online softmax of one page for this lane's row (32 logits, 16 of each
        // token tile), written for latency (nothing runs between its
        // instructions but B's MFMAs): tree reductions for the row max and the
        // row sum, independent exp2 and e4m3 conversions.  Produces the hi and
        // lo e4m3 weight terms (bytes 0-15 from tile 0, 16-31 from tile 1) and
        // d_out, the rescale shift of everything accumulated so far (0 when
        // unchanged); publishes them (d in the sign bits of hi bytes 0 - 7; the
        // own operands stay clean).
        auto softmax_page = [&](f32x16& s0, f32x16& s1, i32x8& ph, i32x8& pl, int& d_out, auto&& between) {
            // row max as a v_max3 tree (fmaxf would first quiet every MFMA
            // result with a v_max x, x, x of its own)
            float q11[11];
#pragma unroll
            for (int g = 0; g < 5; ++g) {
                q11[g] = max3f(s0[3 * g], s0[3 * g + 1], s0[3 * g + 2]);
                q11[5 + g] = max3f(s1[3 * g], s1[3 * g + 1], s1[3 * g + 2]);
            }
            q11[10] = max3f(s0[15], s1[15], q11[0]);
            const float r0 = max3f(q11[1], q11[2], q11[3]), r1 = max3f(q11[4], q11[5], q11[6]),
                        r2 = max3f(q11[7], q11[8], q11[9]);
            const float mx = pair_max(max3f(r0, r1, max3f(r2, q11[10], q11[10]))) * c_exp;
            const bool grow = mx > m + kRescaleSlack8;
            const float m_new = grow ? __builtin_ceilf(mx) : m;
            // (nothing has been accumulated while m is still -inf: no rescale)
            d_out = grow && m != -INFINITY ? (int)fminf(m_new - m, 255.f) : 0;
            m = m_new;
            const float mneg = m == -INFINITY ? 0.f : kWeightOffset8 - m;
            between(0);
            float ps[8];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0[i] = __builtin_fmaf(s0[i], c_exp, mneg);
                s1[i] = __builtin_fmaf(s1[i], c_exp, mneg);
            }
            between(1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0[i] = __builtin_amdgcn_exp2f(s0[i]);
                s1[i] = __builtin_amdgcn_exp2f(s1[i]);
            }
            between(2);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                ps[g] = (s0[4 * g] + s0[4 * g + 1]) + (s0[4 * g + 2] + s0[4 * g + 3]);
                ps[4 + g] = (s1[4 * g] + s1[4 * g + 1]) + (s1[4 * g + 2] + s1[4 * g + 3]);
            }
            l = l * __builtin_ldexpf(1.f, -d_out) +
                (((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7])));
            // (the lo word is built in the register of a value that dies there,
            // so no zero is moved in first)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const f32x16& sv = r < 4 ? s0 : s1;
                const int i0 = 4 * (r & 3);
                const int hw = pack_e4m3(sv[i0], sv[i0 + 1], sv[i0 + 2], sv[i0 + 3]);
                const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
                const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
                ph[r] = hw;
                const float r0 = sv[i0] - h01[0];
                pl[r] = pack_e4m3(r0, sv[i0 + 1] - h01[1], sv[i0 + 2] - h23[0], sv[i0 + 3] - h23[1], __float_as_int(r0));
            }
            const int e0 = ph[0] | spread_nibble(d_out), e1 = ph[1] | spread_nibble(d_out >> 4);
            *(lds_i32x4*)pbuf = (i32x4){e0, e1, ph[2], ph[3]};
            *(lds_i32x4*)(pbuf + 1024) = (i32x4){ph[4], ph[5], ph[6], ph[7]};
            *(lds_i32x4*)(pbuf + 2048) = (i32x4){pl[0], pl[1], pl[2], pl[3]};
            *(lds_i32x4*)(pbuf + 3072) = (i32x4){pl[4], pl[5], pl[6], pl[7]};
        };

        if (pg_begin < pg_end) {
            i32x8 ph_cur, pl_cur;
            int d_cur;
            // both terms of one dim tile of the PV share in one statement,
            // between the wait states after a VALU write of the accumulator
            // (the compiler may copy it) and those before a VALU write may
            // reuse the operand registers
            auto pv_tile = [&](int j, const i32x8& a) {
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\t"
                             "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %3, %0\n\ts_nop 3"
                             : "+v"(o[j]) : "v"(a), "v"(ph_cur), "v"(pl_cur));
            };
            // T(pre): the first page has landed; S and P of it
            lds_sync();
            {
                f32x16 s0, s1;
                qk(pg_begin, s0, s1, [&](int) {});
                if (needs_mask(pg_begin)) mask_s(pg_begin, s0, s1);
                softmax_page(s0, s1, ph_cur, pl_cur, d_cur, [&](int) {});
            }
            for (int k = pg_begin;; ++k) {
                lds_sync();   // T(k)
                const bool more = k + 1 < pg_end;
                if (__builtin_expect(__any(d_cur != 0), 0)) {
                    pv_drain();
                    scale_o(__builtin_ldexpf(1.f, -d_cur));
                }
                // phase 1: PV share of page k (its weights are in registers),
                // then S of page k + 1 (the matrix core is A's alone)
                {
                    lds_u8* cur = slot_ptr(k);
                    i32x8 vf = vfrag(cur, 0);
#pragma unroll
                    for (int j = 0; j < ND; ++j) {
                        pv_tile(j, vf);
                        if (j + 1 < ND) vf = vfrag(cur, j + 1);
                    }
                }
                f32x16 s0, s1;
                if (more) qk(k + 1, s0, s1, [&](int) {});
                lds_sync();   // M(k)
                if (!more) break;
                // phase 2: the softmax of page k + 1 (B's PV of page k keeps the
                // matrix core busy meanwhile); its weights replace those of page k
                if (needs_mask(k + 1)) mask_s(k + 1, s0, s1);
                softmax_page(s0, s1, ph_cur, pl_cur, d_cur, [&](int) {});
                // the wait states between these VALU writes and the next step's MFMAs
                asm volatile("s_nop 1" : "+v"(ph_cur), "+v"(pl_cur));
            }
        }
    } else {
        if (pg_begin < pg_end) {
            // prologue: the first three pages (re-reads past the end), T(pre)
            // once the first has landed
            const int pid0 = page_id(pg_begin);
            const int pid1 = page_id(copy_src(pg_begin + 1));
            const int pid2 = page_id(copy_src(pg_begin + 2));
            copy_page(pg_begin, pid0);
            copy_page(pg_begin + 1, pid1);
            copy_page(pg_begin + 2, pid2);
            int pid_next = page_id(copy_src(pg_begin + 3));
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));
            lds_sync();   // T(pre)
            zero_tail(pg_begin);
            for (int k = pg_begin;; ++k) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));   // page k + 1 has landed
                lds_sync();   // T(k)
                const bool more = k + 1 < pg_end;
                // P(k) first (its latency overlaps the copy issue)
                lds_u8* cur = slot_ptr(k);
                const i32x4 h0 = *(const lds_i32x4*)pbuf;
                const i32x4 h1 = *(const lds_i32x4*)(pbuf + 1024);
                const i32x4 l0 = *(const lds_i32x4*)(pbuf + 2048);
                const i32x4 l1 = *(const lds_i32x4*)(pbuf + 3072);
                copy_page(k + 3, pid_next);
                pid_next = page_id(copy_src(k + 4));
                i32x8 vf[2];
                vf[0] = vfrag(cur, D0);
                vf[1] = vfrag(cur, D0 + 1);
                const int d = gather_nibble(h0[0]) | (gather_nibble(h0[1]) << 4);
                i32x8 ph = (i32x8){h0[0] & 0x7f7f7f7f, h0[1] & 0x7f7f7f7f, h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                i32x8 pl = cat8(l0, l1);
                if (__builtin_expect(__any(d != 0), 0)) {
                    pv_drain();
                    scale_o(__builtin_ldexpf(1.f, -d));
                }
                if (more) zero_tail(k + 1);
                // M(k): P(k) is in registers (the wait covers the reads), A may
                // overwrite it
                lds_sync();
                // the wait states between the VALU writes of ph and an MFMA reading it
                asm volatile("s_nop 1" : "+v"(ph), "+v"(pl));
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    const i32x8 a = vf[j & 1];
                    mfma_o(j, a, ph);
                    mfma_o(j, a, pl);
                    if (j + 2 < ND) vf[j & 1] = vfrag(cur, D0 + j + 2);
                }
                if (!more) break;
            }
        }
    }

    // ---- epilogue: o = kv_scale O / l for this wave's dim tiles of its row
    //      tile; lse = ln(sum exp(s)) for A's rows.
    // No copy may still be writing this workgroup's LDS when it is reused.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    pv_drain();
    const float l_row = pair_sum(l);
    __syncthreads();                      // every wave is done with the ring and the P buffers
    lds_f32* const lbuf = (lds_f32*)(lds + kAb8PBufOff);   // [4 tiles][32 rows]: row sums
    if (A && G == 0) lbuf[s * 32 + lr] = l_row;
    __syncthreads();
    const float lt = lbuf[s * 32 + lr];
    const float inv = lt > 0.f ? kv_scale / lt : 0.f;
    // Rows leave through the idle ring: per half (64 rows, the tiles of SIMDs
    // 2 hf and 2 hf + 1) each wave writes its dims of its rows, scaled, as
    // fp32 (a single piece to an fp32 output) or bf16 (a bf16 output, or a
    // split partial), into rows of 512 e + 16 bytes; then the workgroup stores
    // whole contiguous row pieces, 16 bytes per lane.
    {
        const int tid = wv * 64 + lane;
        const bool f32 = w.nsplit == 1 && !p.out_bf16;
        const int e = f32 ? 4 : 2;
        const int st_row = kV * e + 16;
        const int row_chunks = kV * e / 16;
        uint8_t* gbase = w.nsplit > 1 ? (uint8_t*)p.ws_o + (size_t)w.slot * kMTile * kV * 2
                                      : (uint8_t*)p.out + ((size_t)b * p.rows + (size_t)w.mt * kMTile) * kV * e;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if ((s >> 1) == hf) {
                lds_u8* srow0 = ring + (32 * (s & 1) + lr) * st_row;
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    lds_u8* srow = srow0 + e * (32 * (D0 + j) + 4 * G);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 v = (f32x4){o[j][4 * q4], o[j][4 * q4 + 1], o[j][4 * q4 + 2], o[j][4 * q4 + 3]} * inv;
                        if (f32) {
                            *(__attribute__((address_space(3))) f32x4*)(srow + 4 * 8 * q4) = v;
                        } else {
                            __bf16 __attribute__((ext_vector_type(4))) h;
#pragma unroll
                            for (int i = 0; i < 4; ++i) h[i] = (__bf16)v[i];
                            *(lds_i16x4*)(srow + 2 * 8 * q4) = __builtin_bit_cast(i16x4, h);
                        }
                    }
                }
            }
            __syncthreads();
            for (int i = tid; i < 64 * row_chunks; i += 512) {
                const int rl = i / row_chunks, c = i - rl * row_chunks;
                if (w.mt * kMTile + 64 * hf + rl < p.rows)
                    *(i32x4*)(gbase + (size_t)(64 * hf + rl) * kV * e + 16 * c) =
                        *(const __attribute__((address_space(3))) i32x4*)(ring + rl * st_row + 16 * c);
            }
            __syncthreads();
        }
    }
    if (A && row_ok && G == 0) {
        // l sums exp2(s c - m + 3): ln sum exp = (m - 3 + log2 l) ln 2
        const float lse = l_row > 0.f ? (m - kWeightOffset8 + __log2f(l_row)) * kLn2 : -INFINITY;
        if (w.nsplit == 1) p.lse[(size_t)b * p.rows + row] = lse;
        else p.ws_lse[(size_t)w.slot * kMTile + (row - w.mt * kMTile)] = lse;
    }
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void decode_fp8_ab_kernel(DecodeParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kAb8LdsBytes];
    const WorkItem w = decode_work_item<512>(p, lds);
    if (w.b < 0) return;
    // roles as in the bf16 two-role kernel
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sid = __builtin_amdgcn_readfirstlane(hw_simd_id());
    lds_int* tab = (lds_int*)lds;
    if ((threadIdx.x & 63) == 0) tab[wv] = sid;
    __syncthreads();
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, cnt3 = 0, lower = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int si = __builtin_amdgcn_readfirstlane(tab[i]);
        cnt0 += si == 0; cnt1 += si == 1; cnt2 += si == 2; cnt3 += si == 3;
        lower += (si == sid && i < wv) ? 1 : 0;
    }
    __syncthreads();   // the table's LDS is reused for the pages
    const bool by_hw = cnt0 == 2 && cnt1 == 2 && cnt2 == 2 && cnt3 == 2;
    const bool is_a = by_hw ? lower == 0 : wv < 4;
    const int s = by_hw ? sid : (wv & 3);
    for_each_piece(p, w, [&](const Piece& pc) {
        if (is_a) decode_fp8_ab_body<true>(p, pc, lds, s, wv);
        else decode_fp8_ab_body<false>(p, pc, lds, s, wv);
    });
}

// ---------------------------------------------------------------------------
// LSE merge of one row from n partials: one wave, 8 output dims per lane
// ---------------------------------------------------------------------------
// This lane's 8 consecutive values of a 512-value partial row (fp32 or bf16).
// One lane's 8 values of a partial row, as loaded: fp32 partials (stacked DCP
// shard results) as two f32x4, bf16 split partials as 16 raw bytes that are
// widened only where they are summed, so a group of 8 partials in flight holds
// 32 registers instead of 64.
struct RowF32 {
    f32x4 a, b;
};
__device__ __forceinline__ RowF32 load_row8(const float* row, int lane) {
    const f32x4* src = (const f32x4*)row + 2 * lane;
    return RowF32{src[0], src[1]};
}
__device__ __forceinline__ i32x4 load_row8(const __bf16* row, int lane) {
    return *((const i32x4*)row + lane);
}
__device__ __forceinline__ void add_row8(f32x4& acc0, f32x4& acc1, float w, const RowF32& v) {
    acc0 += w * v.a;
    acc1 += w * v.b;
}
// bf16 element 2j is the low half of dword j, element 2j+1 the high half; a
// bf16 widens to fp32 by taking its 16 bits as the top of the fp32 word.
__device__ __forceinline__ void add_row8(f32x4& acc0, f32x4& acc1, float w, const i32x4& v) {
    const f32x4 a = {__int_as_float(v[0] << 16), __int_as_float(v[0] & 0xffff0000),
                     __int_as_float(v[1] << 16), __int_as_float(v[1] & 0xffff0000)};
    const f32x4 b = {__int_as_float(v[2] << 16), __int_as_float(v[2] & 0xffff0000),
                     __int_as_float(v[3] << 16), __int_as_float(v[3] & 0xffff0000)};
    acc0 += w * a;
    acc1 += w * b;
}

// Running LSE merge state of one row (this lane's 8 output values).
struct MergeAcc {
    float mx, wsum;
    f32x4 acc0, acc1;
};

// Folds partials [i0, i1) of a row into the running state, 8 at a time: all
// loads of a group (8 LSEs, the same address in every lane, and each partial
// row's 8 values of this lane) are issued before any is used, so up to 8
// partials cost one memory round trip.
template <typename PartialAt>
__device__ __forceinline__ void merge_accumulate(MergeAcc& a, int i0, int i1, PartialAt at, int lane) {
    for (int i = i0; i < i1; i += 8) {
        float li[8];
        decltype(load_row8(at.out(0), 0)) v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (i + u < i1) {
                li[u] = *at.lse(i + u);
                v[u] = load_row8(at.out(i + u), lane);
            } else {
                li[u] = -INFINITY;
            }
        }
        float gm = li[0];
#pragma unroll
        for (int u = 1; u < 8; ++u) gm = fmaxf(gm, li[u]);
        if (gm > a.mx) {
            // rescale what is accumulated to the new maximum (nothing yet if
            // mx is still -inf)
            const float r = a.mx == -INFINITY ? 0.f : __expf(a.mx - gm);
            a.acc0 *= r;
            a.acc1 *= r;
            a.wsum *= r;
            a.mx = gm;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // an empty partial (lse -inf) has weight 0 and its output is never
            // read into the sum (it may hold anything)
            if (li[u] != -INFINITY) {
                const float wgt = __expf(li[u] - a.mx);
                a.wsum += wgt;
                add_row8(a.acc0, a.acc1, wgt, v[u]);
            }
        }
    }
}

// Normalises the merged row and stores out (fp32 or bf16) and lse.
__device__ __forceinline__ void merge_finish(const MergeAcc& a, void* out, float* lse_out, size_t orow, int out_bf16,
                                             int lane) {
    const bool empty = a.mx == -INFINITY;
    const float inv = empty ? 0.f : 1.f / a.wsum;
    const f32x4 acc0 = a.acc0 * inv, acc1 = a.acc1 * inv;
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
    if (lane == 0) lse_out[orow] = empty ? -INFINITY : a.mx + __logf(a.wsum);
}

// LSE merge of one row from n partials, by one wave.
template <typename PartialAt>
__device__ __forceinline__ void merge_row(int n, PartialAt at, void* out, float* lse_out, size_t orow,
                                          int out_bf16) {
    const int lane = threadIdx.x & 63;
    MergeAcc a{-INFINITY, 0.f, (f32x4)0.f, (f32x4)0.f};
    merge_accumulate(a, 0, n, at, lane);
    merge_finish(a, out, lse_out, orow, out_bf16, lane);
}

struct SplitPartials {
    const __bf16* ws_o;
    const float* ws_lse;
    int first, mt, m_tiles, rit;
    __device__ const float* lse(int s) const {
        return ws_lse + ((size_t)(first + s) * m_tiles + mt) * kMTile + rit;
    }
    __device__ const __bf16* out(int s) const {
        return ws_o + (((size_t)(first + s) * m_tiles + mt) * kMTile + rit) * kV;
    }
};

// Zero output and -inf LSE: a request with no token (no piece under the
// balanced plan).
__device__ __forceinline__ void write_empty_row(const CombineParams& p, size_t grow, int lane) {
    if (p.out_bf16) {
        *((int4*)((__bf16*)p.out + grow * kV) + lane) = make_int4(0, 0, 0, 0);
    } else {
        f32x4* dst = (f32x4*)((float*)p.out + grow * kV) + 2 * lane;
        dst[0] = (f32x4)0.f;
        dst[1] = (f32x4)0.f;
    }
    if (lane == 0) p.lse[grow] = -INFINITY;
}

// Workgroups of 4 waves in one of two shapes, chosen at launch from how many
// pieces a request is expected to have:
//  - rows_per_wg 4: one wave per output row (few pieces: each wave has all of
//    its row's partials in flight at once);
//  - rows_per_wg 1: the 4 waves share one row, each folding a quarter of its
//    pieces, and their states are merged through LDS (many pieces: 4x the
//    loads in flight per row, and 4x the workgroups to fill the chip).
// Either shape handles any number of pieces.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    __shared__ f32x4 s_acc[4][2][64];
    __shared__ float s_mw[4][2];
    const long long total = (long long)p.batch * p.rows;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool shared_row = p.rows_per_wg == 1;
    const long long grow = shared_row ? (long long)blockIdx.x : (long long)blockIdx.x * 4 + wv;
    if (grow >= total) return;
    const int b = (int)(grow / p.rows);
    const int r = (int)(grow - (long long)b * p.rows);
    const int S = p.req_info[kReqInfoInts * b];
    const int first = p.req_info[kReqInfoInts * b + 1];
    if (S == 1) return;   // a single piece wrote the result directly
    if (S == 0) {
        if (!shared_row || wv == 0) write_empty_row(p, (size_t)grow, lane);
        return;
    }
    // a plan that does not fit the workspace (e.g. one stored for another
    // descriptor) is not followed: every slot index stays below units_max
    if (S < 0 || first < 0 || (long long)(first + S) * p.m_tiles > p.units_max) return;
    SplitPartials at{(const __bf16*)p.ws_o, p.ws_lse, first, r / kMTile, p.m_tiles, r % kMTile};
    MergeAcc a{-INFINITY, 0.f, (f32x4)0.f, (f32x4)0.f};
    if (!shared_row) {
        merge_accumulate(a, 0, S, at, lane);
        merge_finish(a, p.out, p.lse, (size_t)grow, p.out_bf16, lane);
        return;
    }
    // (everything above is uniform over the workgroup, so all 4 waves reach
    // the barrier)
    const int per = (S + 3) / 4;
    const int i0 = min(S, wv * per), i1 = min(S, i0 + per);
    merge_accumulate(a, i0, i1, at, lane);
    s_acc[wv][0][lane] = a.acc0;
    s_acc[wv][1][lane] = a.acc1;
    if (lane == 0) {
        s_mw[wv][0] = a.mx;
        s_mw[wv][1] = a.wsum;
    }
    __syncthreads();
    if (wv != 0) return;
    float mx = s_mw[0][0];
#pragma unroll
    for (int k = 1; k < 4; ++k) mx = fmaxf(mx, s_mw[k][0]);
    MergeAcc m{mx, 0.f, (f32x4)0.f, (f32x4)0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float mk = s_mw[k][0];
        if (mk != -INFINITY) {
            const float f = __expf(mk - mx);
            m.wsum += f * s_mw[k][1];
            m.acc0 += f * s_acc[k][0][lane];
            m.acc1 += f * s_acc[k][1][lane];
        }
    }
    merge_finish(m, p.out, p.lse, (size_t)grow, p.out_bf16, lane);
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
    if (p.plan.group_ok) hipLaunchKernelGGL(decode_bf16_ab_kernel<true>, dim3(units), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL(decode_bf16_ab_kernel<false>, dim3(units), dim3(512), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_after) return hipEventRecord(ev_after, stream);
    return hipSuccess;
}

hipError_t launch_decode_fp8(const DecodeParams& p, int units, hipStream_t stream,
                             hipEvent_t ev_before, hipEvent_t ev_after) {
    if (ev_before) {
        hipError_t e = hipEventRecord(ev_before, stream);
        if (e != hipSuccess) return e;
    }
    clear_stale_error();
    hipLaunchKernelGGL(decode_fp8_ab_kernel, dim3(units), dim3(512), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_after) return hipEventRecord(ev_after, stream);
    return hipSuccess;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
    const long long rows = (long long)p.batch * p.rows;
    if (rows == 0) return hipSuccess;
    clear_stale_error();
    const long long wgs = p.rows_per_wg == 1 ? rows : (rows + 3) / 4;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    clear_stale_error();
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
