// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kQK = 576;          // latent 512 + rope 64
constexpr int kV = 512;           // V = the latent part of the same cache row
constexpr int kPage = 64;         // tokens per cache page
constexpr int kMTile = 128;       // query rows per decode workgroup (heads x query tokens)
constexpr int kTargetUnits = 256; // automatic split: at most this many workgroups (one per CU)
constexpr int kMinChunkPages = 2; // smallest automatic split, in pages
constexpr int kFusedPlanMax = 256; // batches up to this size are planned inside the decode kernel

// The work of one decode workgroup: rows [mt*kMTile, +kMTile) over npages
// cache pages, starting at page page_begin of request b.  With chunk == 0 the
// pages all belong to request b (one piece: a split of the request); with
// chunk > 0 (the balanced plan) they are the global pages [g0, g0 + npages)
// of all requests' pages laid end to end, kv-unit g0 / chunk, and run on
// into the following non-empty requests (one piece per request touched).
// piece is the partial-result index of the first piece (the following ones
// count on from it) and nsplit the number of pieces request b is cut into
// (1: the piece writes the request's result itself).  With chunk == 0 and
// g0 > 1 the item is a group of g0 consecutive splits of request b (forced
// split counts, each split ceil(pages / nsplit) pages but the last), pieces
// piece .. piece + g0 - 1.  b < 0 marks an empty slot.
struct WorkItem {
    int32_t b, mt, piece, page_begin, npages, nsplit, g0, chunk;
};

// One piece of a workgroup's work: rows [mt*kMTile, +kMTile) of request b
// over pages [page_begin, page_end); nsplit == 1 writes out/lse directly,
// otherwise the partial goes to workspace slot `slot` (= piece * m_tiles + mt).
// run > 1: the piece is a group of `run` consecutive splits of the request,
// split j over pages [page_begin + j run_pages, + run_pages) (clipped to
// page_end; the last ones may be empty) with its partial in slot
// slot + j * m_tiles.
struct Piece {
    int32_t b, mt, page_begin, page_end, nsplit, slot;
    int32_t run, run_pages;
};

// Per-request planner output, int32 [batch][kReqInfoInts]: pieces the request
// is cut into (0 for an empty request under the balanced plan), index of its
// first piece, and its first global page (balanced plan; 0 otherwise).
constexpr int kReqInfoInts = 4;

struct PlanParams {
    int32_t batch, rows, m_tiles, max_pages, num_splits, target_units, min_chunk, units_max;
    int32_t balance;            // 1: the balanced plan may be chosen (the kernel runs multi-piece items)
    int32_t group_ok;           // 1: forced splits may be grouped (the kernel instance runs groups)
};

struct DecodeParams {
    const void* q;              // [B][M][576]
    const void* kv;             // [P][64][576]
    const float* kv_scale;      // fp8 only: device float, the per-tensor cache scale
    const int32_t* block_table; // [B][max_pages]
    const int32_t* seq_lens;    // [B]
    const WorkItem* work;       // [units_max] (read when fused_plan == 0)
    WorkItem* work_out;         // the same list (written when fused_plan == 1, one item per workgroup)
    int32_t* req_info;          // [B][kReqInfoInts] (written by workgroup 0 when fused_plan == 1)
    PlanParams plan;            // the planner's inputs (fused_plan == 1)
    int32_t fused_plan;         // 1: every workgroup plans the splits itself (batch <= kFusedPlanMax);
                                // 0: work[] comes from the planner kernel, of this call or an earlier one
    void* out;                  // [B][M][512] of out_dtype
    float* lse;                 // [B][M]
    void* ws_o;                 // bf16 [units_max][kMTile][512] split partials, slot piece * m_tiles + mt
    float* ws_lse;              // [units_max][kMTile]
    float scale_log2;           // scale * log2(e)
    int32_t rows;               // M = q_len * H
    int32_t heads;
    int32_t q_len;
    int32_t causal;
    int32_t max_pages;
    int32_t num_pages;          // pages in the cache pool: every page id is clamped into [0, num_pages)
    int32_t out_bf16;
};

// A block-table entry as a page index that stays inside the pool: one
// unsigned minimum maps a negative or too large id to the last page, so a bad
// entry reads a wrong (but existing) page instead of faulting.
__host__ __device__ inline int clamp_page(int pid, int num_pages) {
    const unsigned int last = (unsigned int)num_pages - 1u;
    return (int)((unsigned int)pid < last ? (unsigned int)pid : last);
}

struct CombineParams {
    const int32_t* req_info;    // [B][kReqInfoInts]: pieces, first piece, first page
    const void* ws_o;           // bf16 split partials
    const float* ws_lse;
    void* out;
    float* lse;
    int32_t batch, rows, m_tiles, out_bf16;
    int32_t units_max;          // slots in ws_o / ws_lse (a split list that needs more is skipped)
    int32_t rows_per_wg;        // 4: one wave per row; 1: the 4 waves of a workgroup share a row
};

struct MergeParams {
    const float* outs;          // [n][rows][512]
    const float* lses;          // [n][rows]
    void* out;
    float* lse;
    int32_t n, rows, out_bf16;
};

// Upper bound on kv-units (request x split, or equal page ranges under the
// balanced plan), and on pieces (at most one more per request), for a descriptor.
inline int64_t kv_units_bound(int batch, int m_tiles, int max_pages, int num_splits) {
    if (num_splits > 0) {
        int64_t per = num_splits < max_pages ? num_splits : max_pages;
        if (per < 1) per = 1;
        return (int64_t)batch * per;
    }
    return (int64_t)kTargetUnits / m_tiles + batch;
}

inline int64_t units_bound(int batch, int m_tiles, int max_pages, int num_splits) {
    int64_t k = kv_units_bound(batch, m_tiles, max_pages, num_splits);
    return ((k + 7) / 8) * 8 * m_tiles;
}

// Bytes of the static device scratch behind mla_decode_partial_noalloc
// (MLA_NOALLOC_SCRATCH_BYTES of the public header).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;

// This device's copy of the static scratch (looked up once per device with
// hipGetSymbolAddress, then reused); nullptr and the HIP error on failure.
hipError_t scratch_for_current_device(void** ptr);

hipError_t launch_plan(const PlanParams& p, const int32_t* seq_lens, int32_t* req_info,
                       WorkItem* work, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, int units, hipStream_t stream,
                              hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_decode_fp8(const DecodeParams& p, int units, hipStream_t stream,
                             hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

}  // namespace mla
