// C ABI of the gfx950 MLA decode library: argument validation, workspace
// layout and kernel launches.  Declarations and contracts: include/mla_decode.h.
#include "mla_decode.h"
#include "mla_decode_timing.h"
#include "mla_internal.h"
#include "mla_qprep.h"
#include "mla_upproj.h"
#include "mla_gather.h"

#include <algorithm>
#include <atomic>
#include <math.h>
#include <stdlib.h>
#include <string.h>

namespace {

// Compute units of the current device (cached per device; the only state the
// library keeps).  The automatic split targets one workgroup per CU, capped at
// kTargetUnits, which also bounds the workspace.
int target_units_for_current_device() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return mla::kTargetUnits;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return mla::kTargetUnits;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus < mla::kTargetUnits ? cus : mla::kTargetUnits;
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Byte offsets of the workspace regions for one descriptor.
struct WorkspaceLayout {
    size_t req_info, work, ws_lse, ws_o, total;
    int64_t units_max;
    int m_tiles;
};

int check_desc(const mla_decode_desc* d) {
    if (!d) return MLA_ERR_INVALID_ARG;
    if (d->batch < 1 || d->q_len < 1 || d->num_heads < 1) return MLA_ERR_INVALID_ARG;
    if (d->num_pages < 1 || d->max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
    if (d->num_splits < 0 || (d->causal != 0 && d->causal != 1)) return MLA_ERR_INVALID_ARG;
    if (d->kv_dtype != MLA_BF16 && d->kv_dtype != MLA_FP8_E4M3) return MLA_ERR_INVALID_ARG;
    if (d->out_dtype != MLA_F32 && d->out_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (d->page_size != MLA_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
    if (d->q_len > 16) return MLA_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)d->q_len * d->num_heads;
    if (rows > (1 << 20)) return MLA_ERR_UNSUPPORTED;
    if ((int64_t)d->max_pages_per_seq * MLA_PAGE_SIZE > INT32_MAX / 2) return MLA_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->max_pages_per_seq > INT32_MAX) return MLA_ERR_UNSUPPORTED;
    if (d->batch > (1 << 20)) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

WorkspaceLayout layout_for(const mla_decode_desc* d) {
    WorkspaceLayout L;
    const int rows = d->q_len * d->num_heads;
    L.m_tiles = (rows + mla::kMTile - 1) / mla::kMTile;
    L.units_max = mla::units_bound(d->batch, L.m_tiles, d->max_pages_per_seq, d->num_splits);
    size_t off = 0;
    L.req_info = off;
    off = align_up(off + sizeof(int32_t) * mla::kReqInfoInts * (size_t)d->batch);
    L.work = off;
    off = align_up(off + sizeof(mla::WorkItem) * (size_t)L.units_max);
    L.ws_lse = off;
    off = align_up(off + sizeof(float) * (size_t)L.units_max * mla::kMTile);
    L.ws_o = off;
    off = align_up(off + sizeof(uint16_t) * (size_t)L.units_max * mla::kMTile * mla::kV);   // bf16 partials
    L.total = off;
    return L;
}

// The descriptor's checks and its workspace layout: every decode entry point
// rejects a descriptor the same way, before looking at any pointer.
int check_layout(const mla_decode_desc* d, WorkspaceLayout* L) {
    const int st = check_desc(d);
    if (st != MLA_OK) return st;
    *L = layout_for(d);
    // work-list slots are 32-bit indices, and each holds kMTile partial rows
    if (L->units_max > INT32_MAX / mla::kMTile) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

// The planner's inputs for one descriptor.
mla::PlanParams plan_params(const mla_decode_desc* d, const WorkspaceLayout& L) {
    mla::PlanParams pp;
    pp.batch = d->batch;
    pp.rows = d->q_len * d->num_heads;
    pp.m_tiles = L.m_tiles;
    pp.max_pages = d->max_pages_per_seq;
    pp.num_splits = d->num_splits;
    pp.target_units = target_units_for_current_device();
    pp.min_chunk = mla::kMinChunkPages;
    pp.units_max = (int32_t)L.units_max;
    // the fp8 kernel runs multi-piece work items (the balanced plan for ragged batches)
    pp.balance = d->kv_dtype == MLA_FP8_E4M3 ? 1 : 0;
    // forced splits that make more work items than one round of workgroups
    // may be grouped (consecutive splits of a request in one workgroup): the
    // two-role bf16 kernel has an instance for such lists
    const int64_t per_req = d->num_splits > 0 ? std::min<int64_t>(d->num_splits, d->max_pages_per_seq) : 0;
    pp.group_ok = d->kv_dtype == MLA_BF16 && per_req > 1 &&
                          (int64_t)d->batch * per_req * L.m_tiles > pp.target_units
                      ? 1
                      : 0;
    return pp;
}

int plan_impl(const mla_decode_desc* d, const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
              void* stream) {
    WorkspaceLayout L;
    const int st = check_layout(d, &L);
    if (st != MLA_OK) return st;
    if (!seq_lens || !aligned(seq_lens, 4)) return MLA_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, kAlign)) return MLA_ERR_WORKSPACE;
    if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    if (mla::launch_plan(plan_params(d, L), seq_lens, (int32_t*)(ws + L.req_info),
                         (mla::WorkItem*)(ws + L.work), (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

// planned: the work list and split counts already sit in the workspace (an
// earlier mla_decode_plan); otherwise this call plans them itself.
int decode_impl(const mla_decode_desc* d, const void* q, const void* kv, const float* kv_scale,
                const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                float* lse, void* workspace, size_t workspace_bytes, void* stream, void* ev0,
                void* ev1, bool planned = false) {
    WorkspaceLayout L;
    const int st = check_layout(d, &L);
    if (st != MLA_OK) return st;
    if (!q || !kv || !block_table || !seq_lens || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4))
        return MLA_ERR_INVALID_ARG;
    if (d->kv_dtype == MLA_FP8_E4M3 ? (kv_scale == nullptr) : (kv_scale != nullptr))
        return MLA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return MLA_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, kAlign)) return MLA_ERR_WORKSPACE;
    if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    int32_t* req_info = (int32_t*)(ws + L.req_info);
    mla::WorkItem* work = (mla::WorkItem*)(ws + L.work);
    const int rows = d->q_len * d->num_heads;

    const mla::PlanParams pp = plan_params(d, L);
    // small batches: every decode workgroup plans the splits itself (one
    // launch fewer); larger ones: one planner workgroup writes the work list;
    // planned calls read the list an earlier planner run left
    const bool fused_plan = !planned && d->batch <= mla::kFusedPlanMax;
    if (!planned && !fused_plan && mla::launch_plan(pp, seq_lens, req_info, work, s) != hipSuccess)
        return MLA_ERR_HIP;

    mla::DecodeParams dp;
    dp.q = q;
    dp.kv = kv;
    dp.kv_scale = kv_scale;
    dp.block_table = block_table;
    dp.seq_lens = seq_lens;
    dp.work = work;
    dp.work_out = work;
    dp.req_info = req_info;
    dp.plan = pp;
    dp.fused_plan = fused_plan ? 1 : 0;
    dp.out = out;
    dp.lse = lse;
    dp.ws_o = ws + L.ws_o;
    dp.ws_lse = (float*)(ws + L.ws_lse);
    dp.scale_log2 = scale * 1.4426950408889634f;
    dp.rows = rows;
    dp.heads = d->num_heads;
    dp.q_len = d->q_len;
    dp.causal = d->q_len > 1 ? d->causal : 0;
    dp.max_pages = d->max_pages_per_seq;
    dp.num_pages = d->num_pages;
    dp.out_bf16 = d->out_dtype == MLA_BF16;
    const hipError_t de = d->kv_dtype == MLA_FP8_E4M3
                              ? mla::launch_decode_fp8(dp, (int)L.units_max, s, (hipEvent_t)ev0, (hipEvent_t)ev1)
                              : mla::launch_decode_bf16(dp, (int)L.units_max, s, (hipEvent_t)ev0, (hipEvent_t)ev1);
    if (de != hipSuccess) return MLA_ERR_HIP;

    mla::CombineParams cp;
    cp.req_info = req_info;
    cp.ws_o = dp.ws_o;
    cp.ws_lse = dp.ws_lse;
    cp.out = out;
    cp.lse = lse;
    cp.batch = d->batch;
    cp.rows = rows;
    cp.m_tiles = L.m_tiles;
    cp.out_bf16 = dp.out_bf16;
    cp.units_max = (int32_t)L.units_max;
    // pieces a full-length request gets: the forced split count, or the
    // automatic target spread over every request and row tile; with more than
    // 8 the 4 waves of a combine workgroup share one row
    const int64_t pieces_hint = d->num_splits > 0
                                    ? std::min<int64_t>(d->num_splits, d->max_pages_per_seq)
                                    : pp.target_units / std::max<int64_t>(1, (int64_t)d->batch * L.m_tiles);
    cp.rows_per_wg = pieces_hint > 8 ? 1 : 4;
    if (mla::launch_combine(cp, s) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_workspace_size(const mla_decode_desc* desc, size_t* bytes) {
    if (!bytes) return MLA_ERR_INVALID_ARG;
    WorkspaceLayout L;
    const int st = check_layout(desc, &L);
    if (st != MLA_OK) return st;
    *bytes = L.total;
    return MLA_OK;
}

int mla_decode_partial(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                       const float* kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                       float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
    return decode_impl(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse,
                       workspace, workspace_bytes, stream, nullptr, nullptr);
}

int mla_decode_partial_timed(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                             const float* kv_scale, const int32_t* block_table,
                             const int32_t* seq_lens, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* event_before_decode, void* event_after_decode) {
    return decode_impl(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse,
                       workspace, workspace_bytes, stream, event_before_decode, event_after_decode);
}

int mla_decode_partial_noalloc(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                               const float* kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                               float scale, void* out, float* lse, void* stream) {
    static_assert(mla::kNoAllocScratchBytes == MLA_NOALLOC_SCRATCH_BYTES, "scratch size");
    WorkspaceLayout L;
    const int st = check_layout(desc, &L);
    if (st != MLA_OK) return st;
    if (L.total > mla::kNoAllocScratchBytes) return MLA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (mla::scratch_for_current_device(&ws) != hipSuccess) return MLA_ERR_HIP;
    return decode_impl(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse, ws,
                       mla::kNoAllocScratchBytes, stream, nullptr, nullptr);
}

int mla_decode_plan(const mla_decode_desc* desc, const int32_t* seq_lens, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return plan_impl(desc, seq_lens, workspace, workspace_bytes, stream);
}

int mla_decode_partial_planned(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                               const float* kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                               float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return decode_impl(desc, q, kv_cache, kv_scale, block_table, seq_lens, scale, out, lse,
                       workspace, workspace_bytes, stream, nullptr, nullptr, true);
}

int mla_merge_states(const float* outs, const float* lses, int32_t n, int32_t rows, void* out,
                     float* lse, int32_t out_dtype, void* stream) {
    if (n < 1 || n > 4096 || rows < 0) return MLA_ERR_INVALID_ARG;
    if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (rows == 0) return MLA_OK;
    if (!outs || !lses || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (!aligned(outs, 16) || !aligned(out, 16) || !aligned(lses, 4) || !aligned(lse, 4))
        return MLA_ERR_INVALID_ARG;
    mla::MergeParams mp;
    mp.outs = outs;
    mp.lses = lses;
    mp.out = out;
    mp.lse = lse;
    mp.n = n;
    mp.rows = rows;
    mp.out_bf16 = out_dtype == MLA_BF16;
    if (mla::launch_merge(mp, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_query_prep(const mla_query_prep_desc* d, const void* q_nope, const void* q_pe,
                   const void* w_uk, const float* q_scale, void* q_out, void* stream) {
    if (!d) return MLA_ERR_INVALID_ARG;
    if (d->rows < 0 || d->num_heads < 1) return MLA_ERR_INVALID_ARG;
    if (d->out_dtype != MLA_BF16 && d->out_dtype != MLA_FP8_E4M3) return MLA_ERR_INVALID_ARG;
    if (d->nope_dim < 16 || d->nope_dim > 256 || d->nope_dim % 16 != 0) return MLA_ERR_UNSUPPORTED;
    if (d->num_heads > (1 << 16) || (int64_t)d->rows * d->num_heads > (int64_t)1 << 28) return MLA_ERR_UNSUPPORTED;
    if ((d->out_dtype == MLA_FP8_E4M3) != (q_scale != nullptr)) return MLA_ERR_INVALID_ARG;
    if (d->rows == 0) return MLA_OK;
    if (!q_nope || !q_pe || !w_uk || !q_out) return MLA_ERR_INVALID_ARG;
    if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(q_out, 16) ||
        (q_scale && !aligned(q_scale, 4)))
        return MLA_ERR_INVALID_ARG;
    mla::QueryPrepParams p;
    p.q_nope = q_nope;
    p.q_pe = q_pe;
    p.w_uk = w_uk;
    p.q_scale = q_scale;
    p.q_out = q_out;
    p.rows = d->rows;
    p.heads = d->num_heads;
    p.nope_dim = d->nope_dim;
    p.out_fp8 = d->out_dtype == MLA_FP8_E4M3;
    if (mla::launch_query_prep(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_up_project(const mla_up_project_desc* d, const void* o_lat, const void* w_uv, void* out,
                   void* stream) {
    if (!d) return MLA_ERR_INVALID_ARG;
    if (d->rows < 0 || d->num_heads < 1) return MLA_ERR_INVALID_ARG;
    if ((d->in_dtype != MLA_F32 && d->in_dtype != MLA_BF16) || (d->out_dtype != MLA_F32 && d->out_dtype != MLA_BF16))
        return MLA_ERR_INVALID_ARG;
    if (d->v_head_dim < 32 || d->v_head_dim > 512 || d->v_head_dim % 32 != 0) return MLA_ERR_UNSUPPORTED;
    if (d->num_heads > (1 << 16) || (int64_t)d->rows * d->num_heads > (int64_t)1 << 26) return MLA_ERR_UNSUPPORTED;
    if (d->rows == 0) return MLA_OK;
    if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
    if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
    mla::UpProjParams p;
    p.o_lat = o_lat;
    p.lses = nullptr;
    p.lse_out = nullptr;
    p.w_uv = w_uv;
    p.out = out;
    p.rows = d->rows;
    p.heads = d->num_heads;
    p.vdim = d->v_head_dim;
    p.in_f32 = d->in_dtype == MLA_F32;
    p.out_f32 = d->out_dtype == MLA_F32;
    p.n_merge = 0;
    if (mla::launch_up_project(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_merge_up_project(const float* outs, const float* lses, int32_t n, const mla_up_project_desc* d,
                         const void* w_uv, void* out, float* lse, void* stream) {
    if (!d) return MLA_ERR_INVALID_ARG;
    if (n < 1 || n > mla::kMaxMergeUp) return MLA_ERR_INVALID_ARG;
    if (d->rows < 0 || d->num_heads < 1 || d->in_dtype != MLA_F32) return MLA_ERR_INVALID_ARG;
    if (d->out_dtype != MLA_F32 && d->out_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (d->v_head_dim < 32 || d->v_head_dim > 512 || d->v_head_dim % 32 != 0) return MLA_ERR_UNSUPPORTED;
    if (d->num_heads > (1 << 16) || (int64_t)d->rows * d->num_heads > (int64_t)1 << 26) return MLA_ERR_UNSUPPORTED;
    if (d->rows == 0) return MLA_OK;
    if (!outs || !lses || !w_uv || !out) return MLA_ERR_INVALID_ARG;
    if (!aligned(outs, 16) || !aligned(w_uv, 16) || !aligned(out, 16) || !aligned(lses, 4) || (lse && !aligned(lse, 4)))
        return MLA_ERR_INVALID_ARG;
    mla::UpProjParams p;
    p.o_lat = outs;
    p.lses = lses;
    p.lse_out = lse;
    p.w_uv = w_uv;
    p.out = out;
    p.rows = d->rows;
    p.heads = d->num_heads;
    p.vdim = d->v_head_dim;
    p.in_f32 = 1;
    p.out_f32 = d->out_dtype == MLA_F32;
    p.n_merge = n;
    if (mla::launch_up_project(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_gather_cache(const void* kv_cache, int32_t kv_dtype, const float* kv_scale,
                     const int32_t* block_table, int32_t batch, int32_t num_pages,
                     int32_t max_pages_per_seq, const int32_t* seq_starts, const int32_t* cu_lens,
                     int64_t total_rows, void* out, void* stream) {
    if (kv_dtype != MLA_BF16 && kv_dtype != MLA_FP8_E4M3) return MLA_ERR_INVALID_ARG;
    if (batch < 1 || num_pages < 1 || max_pages_per_seq < 1 || total_rows < 0) return MLA_ERR_INVALID_ARG;
    if ((kv_dtype == MLA_FP8_E4M3) != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
    if ((int64_t)batch * max_pages_per_seq > INT32_MAX || total_rows > ((int64_t)1 << 34)) return MLA_ERR_UNSUPPORTED;
    if (total_rows == 0) return MLA_OK;
    if (!kv_cache || !block_table || !seq_starts || !cu_lens || !out) return MLA_ERR_INVALID_ARG;
    if (!aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(block_table, 4) || !aligned(seq_starts, 4) ||
        !aligned(cu_lens, 4) || (kv_scale && !aligned(kv_scale, 4)))
        return MLA_ERR_INVALID_ARG;
    mla::GatherParams p;
    p.kv = kv_cache;
    p.kv_scale = kv_scale;
    p.block_table = block_table;
    p.seq_starts = seq_starts;
    p.cu_lens = cu_lens;
    p.out = out;
    p.total_rows = total_rows;
    p.batch = batch;
    p.num_pages = num_pages;
    p.max_pages = max_pages_per_seq;
    p.fp8 = kv_dtype == MLA_FP8_E4M3;
    if (mla::launch_gather_cache(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_merge_two_states(int32_t rows, int32_t head_dim, int32_t in_dtype, int32_t out_dtype,
                         const void* prefix_out, const float* prefix_lse, const void* suffix_out,
                         const float* suffix_lse, void* out, float* lse, void* stream) {
    if (rows < 0 || head_dim < 4 || head_dim > 4096 || head_dim % 4 != 0) return MLA_ERR_INVALID_ARG;
    if ((in_dtype != MLA_F32 && in_dtype != MLA_BF16) || (out_dtype != MLA_F32 && out_dtype != MLA_BF16))
        return MLA_ERR_INVALID_ARG;
    if ((int64_t)rows * head_dim > ((int64_t)1 << 32)) return MLA_ERR_UNSUPPORTED;
    if (rows == 0) return MLA_OK;
    if (!prefix_out || !prefix_lse || !suffix_out || !suffix_lse || !out) return MLA_ERR_INVALID_ARG;
    if (!aligned(prefix_out, 16) || !aligned(suffix_out, 16) || !aligned(out, 16) || !aligned(prefix_lse, 4) ||
        !aligned(suffix_lse, 4) || (lse && !aligned(lse, 4)))
        return MLA_ERR_INVALID_ARG;
    mla::MergeTwoParams p;
    p.prefix_out = prefix_out;
    p.prefix_lse = prefix_lse;
    p.suffix_out = suffix_out;
    p.suffix_lse = suffix_lse;
    p.out = out;
    p.lse = lse;
    p.rows = rows;
    p.head_dim = head_dim;
    p.in_f32 = in_dtype == MLA_F32;
    p.out_f32 = out_dtype == MLA_F32;
    if (mla::launch_merge_two(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "ok";
        case MLA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or shape)";
        case MLA_ERR_UNSUPPORTED: return "unsupported combination (page size, q_len, dtype or size limit)";
        case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MLA_ERR_HIP: return "HIP runtime error or kernel launch failure";
        case MLA_ERR_SCRATCH_LIMIT:
            return "the descriptor needs more workspace than the static scratch (MLA_NOALLOC_SCRATCH_BYTES) "
                   "holds; use mla_decode_partial with a caller workspace";
        default: return "unknown status";
    }
}

}  // extern "C"
