// Host-only stand-ins for the gfx950 kernel launchers and the two HIP runtime
// queries the C-ABI layer makes, for a sanitizer build of that layer on a
// machine without a GPU.  Each launcher checks that every buffer the kernel
// would touch, at the extent its parameter block implies, lies inside a buffer
// the driver registered (the caller's arguments), then counts the launch.
#include "mla_internal.h"
#include "mla_gather.h"
#include "mla_qprep.h"
#include "mla_upproj.h"

#include "sanitize_harness.h"

#include <stdio.h>
#include <stdlib.h>

namespace {

struct Region {
    const char* name;
    uintptr_t lo, hi;
};
Region g_regions[64];
int g_nregions = 0;
int g_launches = 0;
int g_failures = 0;

void fail(const char* kernel, const char* what, const void* p, size_t bytes) {
    fprintf(stderr, "STUB FAILURE: %s: %s [%p, +%zu) is outside every registered buffer\n", kernel, what, p, bytes);
    ++g_failures;
}

// [p, p + bytes) inside one registered buffer (an empty extent always passes)
void need(const char* kernel, const char* what, const void* p, size_t bytes) {
    if (bytes == 0) return;
    const uintptr_t a = (uintptr_t)p;
    for (int i = 0; i < g_nregions; ++i)
        if (a >= g_regions[i].lo && a <= g_regions[i].hi && bytes <= g_regions[i].hi - a) return;
    fail(kernel, what, p, bytes);
}

void expect(const char* kernel, bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "STUB FAILURE: %s: %s\n", kernel, what);
        ++g_failures;
    }
}

}  // namespace

void harness_register(const char* name, const void* p, size_t bytes) {
    if (g_nregions == 64) abort();
    g_regions[g_nregions++] = Region{name, (uintptr_t)p, (uintptr_t)p + bytes};
}
void harness_clear() { g_nregions = 0; }
int harness_launches() { return g_launches; }
int harness_failures() { return g_failures; }

// ---- the HIP runtime queries of the C-ABI layer
extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev) {
    (void)dev;
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

namespace mla {

// the static scratch: a registered host buffer of the same size
hipError_t scratch_for_current_device(void** ptr) {
    static uint8_t* buf = nullptr;
    if (!buf) buf = (uint8_t*)aligned_alloc(256, kNoAllocScratchBytes);
    harness_register("static scratch", buf, kNoAllocScratchBytes);
    *ptr = buf;
    return hipSuccess;
}

static void check_decode(const char* k, const DecodeParams& p, int units) {
    expect(k, units > 0 && units == p.plan.units_max, "grid size differs from the planner's slot count");
    expect(k, p.plan.m_tiles == (p.rows + kMTile - 1) / kMTile, "row tiles");
    expect(k, p.num_pages >= 1 && p.max_pages >= 1, "page counts");
    const size_t e = p.kv_scale ? 1 : 2;
    const size_t B = (size_t)p.plan.batch;
    need(k, "q", p.q, B * p.rows * kQK * e);
    need(k, "kv", p.kv, (size_t)p.num_pages * kPage * kQK * e);
    if (p.kv_scale) need(k, "kv_scale", p.kv_scale, 4);
    need(k, "block_table", p.block_table, B * p.max_pages * 4);
    need(k, "seq_lens", p.seq_lens, B * 4);
    need(k, "work", p.work, (size_t)units * sizeof(WorkItem));
    need(k, "work_out", p.work_out, (size_t)units * sizeof(WorkItem));
    need(k, "req_info", p.req_info, B * 4 * kReqInfoInts);
    need(k, "out", p.out, B * p.rows * kV * (p.out_bf16 ? 2 : 4));
    need(k, "lse", p.lse, B * p.rows * 4);
    need(k, "ws_o", p.ws_o, (size_t)units * kMTile * kV * 2);
    need(k, "ws_lse", p.ws_lse, (size_t)units * kMTile * 4);
    ++g_launches;
}

hipError_t launch_plan(const PlanParams& p, const int32_t* seq_lens, int32_t* req_info, WorkItem* work,
                       hipStream_t) {
    need("plan", "seq_lens", seq_lens, (size_t)p.batch * 4);
    need("plan", "req_info", req_info, (size_t)p.batch * 4 * kReqInfoInts);
    need("plan", "work", work, (size_t)p.units_max * sizeof(WorkItem));
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeParams& p, int units, hipStream_t, hipEvent_t, hipEvent_t) {
    expect("decode_bf16", p.kv_scale == nullptr, "bf16 decode with a kv_scale");
    check_decode("decode_bf16", p, units);
    return hipSuccess;
}

hipError_t launch_decode_fp8(const DecodeParams& p, int units, hipStream_t, hipEvent_t, hipEvent_t) {
    expect("decode_fp8", p.kv_scale != nullptr, "fp8 decode without a kv_scale");
    check_decode("decode_fp8", p, units);
    return hipSuccess;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t) {
    const size_t B = (size_t)p.batch;
    need("combine", "req_info", p.req_info, B * 4 * kReqInfoInts);
    need("combine", "ws_o", p.ws_o, (size_t)p.units_max * kMTile * kV * 2);
    need("combine", "ws_lse", p.ws_lse, (size_t)p.units_max * kMTile * 4);
    need("combine", "out", p.out, B * p.rows * kV * (p.out_bf16 ? 2 : 4));
    need("combine", "lse", p.lse, B * p.rows * 4);
    expect("combine", p.rows_per_wg == 1 || p.rows_per_wg == 4, "rows_per_wg is neither 1 nor 4");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t) {
    const size_t n = (size_t)p.n, R = (size_t)p.rows;
    need("merge", "outs", p.outs, n * R * kV * 4);
    need("merge", "lses", p.lses, n * R * 4);
    need("merge", "out", p.out, R * kV * (p.out_bf16 ? 2 : 4));
    need("merge", "lse", p.lse, R * 4);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_query_prep(const QueryPrepParams& p, hipStream_t) {
    const size_t RH = (size_t)p.rows * p.heads;
    need("query_prep", "q_nope", p.q_nope, RH * p.nope_dim * 2);
    need("query_prep", "q_pe", p.q_pe, RH * 64 * 2);
    need("query_prep", "w_uk", p.w_uk, (size_t)p.heads * 512 * p.nope_dim * 2);
    if (p.out_fp8) need("query_prep", "q_scale", p.q_scale, 4);
    need("query_prep", "q_out", p.q_out, RH * kQK * (p.out_fp8 ? 1 : 2));
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_up_project(const UpProjParams& p, hipStream_t) {
    const size_t RH = (size_t)p.rows * p.heads;
    if (p.n_merge > 0) {
        need("up_project", "partials", p.o_lat, (size_t)p.n_merge * RH * kV * 4);
        need("up_project", "lses", p.lses, (size_t)p.n_merge * RH * 4);
        if (p.lse_out) need("up_project", "lse_out", p.lse_out, RH * 4);
    } else {
        need("up_project", "o_lat", p.o_lat, RH * kV * (p.in_f32 ? 4 : 2));
    }
    need("up_project", "w_uv", p.w_uv, (size_t)p.heads * p.vdim * kV * 2);
    need("up_project", "out", p.out, RH * p.vdim * (p.out_f32 ? 4 : 2));
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_gather_cache(const GatherParams& p, hipStream_t) {
    const size_t e = p.fp8 ? 1 : 2;
    need("gather", "kv", p.kv, (size_t)p.num_pages * kPage * kQK * e);
    if (p.fp8) need("gather", "kv_scale", p.kv_scale, 4);
    need("gather", "block_table", p.block_table, (size_t)p.batch * p.max_pages * 4);
    need("gather", "seq_starts", p.seq_starts, (size_t)p.batch * 4);
    need("gather", "cu_lens", p.cu_lens, ((size_t)p.batch + 1) * 4);
    need("gather", "out", p.out, (size_t)p.total_rows * kQK * 2);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_merge_two(const MergeTwoParams& p, hipStream_t) {
    const size_t n = (size_t)p.rows * p.head_dim;
    need("merge_two", "prefix_out", p.prefix_out, n * (p.in_f32 ? 4 : 2));
    need("merge_two", "suffix_out", p.suffix_out, n * (p.in_f32 ? 4 : 2));
    need("merge_two", "prefix_lse", p.prefix_lse, (size_t)p.rows * 4);
    need("merge_two", "suffix_lse", p.suffix_lse, (size_t)p.rows * 4);
    need("merge_two", "out", p.out, n * (p.out_f32 ? 4 : 2));
    if (p.lse) need("merge_two", "lse", p.lse, (size_t)p.rows * 4);
    ++g_launches;
    return hipSuccess;
}

}  // namespace mla
