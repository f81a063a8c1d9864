// Boundary cases of the C ABI, run against a host-only build of its validation
// layer (the kernel launchers replaced by stand-ins that check every extent a
// kernel would touch).  Built with AddressSanitizer and UndefinedBehaviorSanitizer
// by the CPU test suite; exits non-zero on any failed check.
//
// Device pointers are stood in for by host buffers: the layer never
// dereferences them, it only checks and forwards them.
#include "mla_decode.h"
#include "mla_decode_timing.h"

#include "sanitize_harness.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

static int g_fails = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c);        \
            ++g_fails;                                                             \
        }                                                                          \
    } while (0)

namespace {

// A registered stand-in buffer of exactly `bytes` (256-byte aligned start).
struct Buf {
    uint8_t* p = nullptr;
    size_t n = 0;
    Buf(const char* name, size_t bytes) : n(bytes) {
        p = (uint8_t*)aligned_alloc(256, bytes ? (bytes + 255) / 256 * 256 : 256);
        memset(p, 0, bytes ? bytes : 1);
        harness_register(name, p, bytes);
    }
    ~Buf() { free(p); }
    Buf(const Buf&) = delete;
    Buf& operator=(const Buf&) = delete;
};

mla_decode_desc desc(int batch, int q_len, int heads, int num_pages, int max_pages, int kv_dtype = MLA_BF16,
                     int out_dtype = MLA_F32, int causal = 0, int num_splits = 0) {
    mla_decode_desc d;
    d.batch = batch;
    d.q_len = q_len;
    d.num_heads = heads;
    d.page_size = MLA_PAGE_SIZE;
    d.num_pages = num_pages;
    d.max_pages_per_seq = max_pages;
    d.kv_dtype = kv_dtype;
    d.out_dtype = out_dtype;
    d.causal = causal;
    d.num_splits = num_splits;
    return d;
}

// Every argument buffer of one decode call, sized from the descriptor.
struct DecodeArgs {
    mla_decode_desc d;
    size_t ws_bytes = 0;
    Buf *q, *kv, *kvs, *bt, *sl, *out, *lse, *ws;
    explicit DecodeArgs(const mla_decode_desc& dd) : d(dd) {
        harness_clear();
        const size_t e = d.kv_dtype == MLA_FP8_E4M3 ? 1 : 2;
        const size_t rows = (size_t)d.batch * d.q_len * d.num_heads;
        CHECK(mla_decode_workspace_size(&d, &ws_bytes) == MLA_OK);
        q = new Buf("q", rows * MLA_QK_DIM * e);
        kv = new Buf("kv", (size_t)d.num_pages * MLA_PAGE_SIZE * MLA_QK_DIM * e);
        kvs = new Buf("kv_scale", 4);
        bt = new Buf("block_table", (size_t)d.batch * d.max_pages_per_seq * 4);
        sl = new Buf("seq_lens", (size_t)d.batch * 4);
        out = new Buf("out", rows * MLA_LATENT_DIM * (d.out_dtype == MLA_F32 ? 4 : 2));
        lse = new Buf("lse", rows * 4);
        ws = new Buf("workspace", ws_bytes);
    }
    ~DecodeArgs() {
        delete q; delete kv; delete kvs; delete bt; delete sl; delete out; delete lse; delete ws;
        harness_clear();
    }
    const float* scale_ptr() const { return d.kv_dtype == MLA_FP8_E4M3 ? (const float*)kvs->p : nullptr; }
    int call(float scale = 0.125f) {
        return mla_decode_partial(&d, q->p, kv->p, scale_ptr(), (const int32_t*)bt->p, (const int32_t*)sl->p,
                                  scale, out->p, (float*)lse->p, ws->p, ws_bytes, nullptr);
    }
};

// status of a call, and that it enqueued `launches` kernels (0 on any error)
void expect_call(int status, int want, int launches_before, int launches) {
    CHECK(status == want);
    CHECK(harness_launches() - launches_before == (want == MLA_OK ? launches : 0));
}

void decode_cases() {
    // good calls of several shapes: plan fused into the decode (<= 256
    // requests) or a separate planner launch, then decode and combine
    const mla_decode_desc good[] = {
        desc(2, 1, 16, 6, 2), desc(64, 1, 128, 4096, 64), desc(4, 2, 128, 8192, 2048, MLA_BF16, MLA_F32, 1),
        desc(128, 1, 128, 17714, 256, MLA_FP8_E4M3), desc(32, 1, 512, 4096, 128, MLA_BF16, MLA_BF16),
        desc(300, 1, 128, 600, 2), desc(4, 2, 128, 8192, 2048, MLA_BF16, MLA_F32, 1, 256),
        desc(3, 16, 64, 10, 4, MLA_FP8_E4M3, MLA_BF16, 1, 3)};
    for (const auto& g : good) {
        DecodeArgs a(g);
        int before = harness_launches();
        expect_call(a.call(), MLA_OK, before, g.batch > 256 ? 3 : 2);
        before = harness_launches();
        expect_call(mla_decode_partial_timed(&a.d, a.q->p, a.kv->p, a.scale_ptr(), (const int32_t*)a.bt->p,
                                             (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, a.ws->p,
                                             a.ws_bytes, nullptr, nullptr, nullptr),
                    MLA_OK, before, g.batch > 256 ? 3 : 2);
        before = harness_launches();
        expect_call(mla_decode_plan(&a.d, (const int32_t*)a.sl->p, a.ws->p, a.ws_bytes, nullptr), MLA_OK, before, 1);
        before = harness_launches();
        expect_call(mla_decode_partial_planned(&a.d, a.q->p, a.kv->p, a.scale_ptr(), (const int32_t*)a.bt->p,
                                               (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, a.ws->p,
                                               a.ws_bytes, nullptr),
                    MLA_OK, before, 2);
    }

    // argument errors: each returns its status before any launch
    DecodeArgs a(desc(2, 1, 16, 6, 2));
    const int32_t* bt = (const int32_t*)a.bt->p;
    const int32_t* sl = (const int32_t*)a.sl->p;
    float* lse = (float*)a.lse->p;
    int b = harness_launches();
    expect_call(mla_decode_partial(nullptr, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    const void* nul = nullptr;
    expect_call(mla_decode_partial(&a.d, nul, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p, a.ws_bytes,
                                   nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, nul, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p, a.ws_bytes,
                                   nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, nullptr, sl, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, nullptr, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, nullptr, lse, a.ws->p, a.ws_bytes,
                                   nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, nullptr, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    // misaligned pointers (q, kv, out need 16 bytes; lse, block table, seq_lens 4)
    expect_call(mla_decode_partial(&a.d, a.q->p + 8, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p + 2, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p + 4, lse, a.ws->p,
                                   a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, (float*)(a.lse->p + 2),
                                   a.ws->p, a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, (const int32_t*)(a.bt->p + 1), sl, 0.1f,
                                   a.out->p, lse, a.ws->p, a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, (const int32_t*)(a.sl->p + 3), 0.1f,
                                   a.out->p, lse, a.ws->p, a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    // a kv_scale with a bf16 cache
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, (const float*)a.kvs->p, bt, sl, 0.1f, a.out->p, lse,
                                   a.ws->p, a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);
    // softmax scales that are not finite and positive
    for (float s : {0.f, -1.f, NAN, INFINITY, -0.f})
        expect_call(a.call(s), MLA_ERR_INVALID_ARG, b, 0);
    // workspace: missing, misaligned, one byte short
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, nullptr,
                                   a.ws_bytes, nullptr), MLA_ERR_WORKSPACE, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p + 16,
                                   a.ws_bytes, nullptr), MLA_ERR_WORKSPACE, b, 0);
    expect_call(mla_decode_partial(&a.d, a.q->p, a.kv->p, nullptr, bt, sl, 0.1f, a.out->p, lse, a.ws->p,
                                   a.ws_bytes - 1, nullptr), MLA_ERR_WORKSPACE, b, 0);
    expect_call(mla_decode_plan(&a.d, sl, a.ws->p, a.ws_bytes - 1, nullptr), MLA_ERR_WORKSPACE, b, 0);
    expect_call(mla_decode_plan(&a.d, nullptr, a.ws->p, a.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, b, 0);

    // an fp8 cache without its scale
    {
        DecodeArgs f(desc(2, 1, 16, 6, 2, MLA_FP8_E4M3));
        int bb = harness_launches();
        expect_call(mla_decode_partial(&f.d, f.q->p, f.kv->p, nullptr, (const int32_t*)f.bt->p,
                                       (const int32_t*)f.sl->p, 0.1f, f.out->p, (float*)f.lse->p, f.ws->p,
                                       f.ws_bytes, nullptr), MLA_ERR_INVALID_ARG, bb, 0);
    }
}

// the allocation-free decode: good descriptors run on the static scratch,
// one that needs more returns MLA_ERR_SCRATCH_LIMIT before any launch
void noalloc_cases() {
    const mla_decode_desc fits[] = {desc(64, 1, 128, 4096, 64), desc(128, 1, 128, 17714, 256, MLA_FP8_E4M3),
                                    desc(32, 1, 512, 4096, 128), desc(4, 2, 128, 8192, 2048, MLA_BF16, MLA_F32, 1),
                                    desc(240, 1, 128, 600, 2), desc(300, 1, 128, 600, 2),
                                    desc(760, 1, 128, 600, 2)};   // 1,016 units: the most that fit
    for (const auto& g : fits) {
        DecodeArgs a(g);
        CHECK(a.ws_bytes <= MLA_NOALLOC_SCRATCH_BYTES);
        const int b = harness_launches();
        expect_call(mla_decode_partial_noalloc(&a.d, a.q->p, a.kv->p, a.scale_ptr(), (const int32_t*)a.bt->p,
                                               (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, nullptr),
                    MLA_OK, b, g.batch > 256 ? 3 : 2);
    }
    const mla_decode_desc too_big[] = {desc(4, 2, 128, 8192, 2048, MLA_BF16, MLA_F32, 1, 256),
                                       desc(768, 1, 128, 600, 2),   // 1,024 units
                                       desc(1024, 1, 128, 4096, 8)};
    for (const auto& g : too_big) {
        DecodeArgs a(g);
        CHECK(a.ws_bytes > MLA_NOALLOC_SCRATCH_BYTES);
        const int b = harness_launches();
        expect_call(mla_decode_partial_noalloc(&a.d, a.q->p, a.kv->p, a.scale_ptr(), (const int32_t*)a.bt->p,
                                               (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, nullptr),
                    MLA_ERR_SCRATCH_LIMIT, b, 0);
    }
    DecodeArgs a(desc(2, 1, 16, 6, 2));
    const int b = harness_launches();
    expect_call(mla_decode_partial_noalloc(&a.d, nullptr, a.kv->p, nullptr, (const int32_t*)a.bt->p,
                                           (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, nullptr),
                MLA_ERR_INVALID_ARG, b, 0);
    expect_call(mla_decode_partial_noalloc(nullptr, a.q->p, a.kv->p, nullptr, (const int32_t*)a.bt->p,
                                           (const int32_t*)a.sl->p, 0.1f, a.out->p, (float*)a.lse->p, nullptr),
                MLA_ERR_INVALID_ARG, b, 0);
}

void descriptor_cases() {
    size_t n = 0;
    struct Bad {
        mla_decode_desc d;
        int status;
    };
    mla_decode_desc base = desc(2, 1, 16, 6, 2);
    auto with = [&](auto f) {
        mla_decode_desc d = base;
        f(d);
        return d;
    };
    const Bad bad[] = {
        {with([](mla_decode_desc& d) { d.batch = 0; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.batch = -5; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.q_len = 0; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.q_len = 17; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.num_heads = 0; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.page_size = 32; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.num_pages = 0; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.max_pages_per_seq = 0; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.kv_dtype = MLA_F32; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.kv_dtype = 7; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.out_dtype = MLA_FP8_E4M3; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.causal = 2; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.num_splits = -1; }), MLA_ERR_INVALID_ARG},
        {with([](mla_decode_desc& d) { d.num_heads = (1 << 20) + 1; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.q_len = 16; d.num_heads = (1 << 16) + 1; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.batch = (1 << 20) + 1; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.max_pages_per_seq = INT32_MAX; }), MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.batch = 1 << 20; d.max_pages_per_seq = 1 << 12; }), MLA_ERR_UNSUPPORTED},
        // work lists too long for 32-bit slot indices
        {with([](mla_decode_desc& d) { d.batch = 1 << 19; d.max_pages_per_seq = 4096; d.num_splits = 4096; }),
         MLA_ERR_UNSUPPORTED},
        {with([](mla_decode_desc& d) { d.batch = 1 << 20; d.num_heads = 1 << 20; }), MLA_ERR_UNSUPPORTED},
    };
    for (const auto& c : bad) {
        CHECK(mla_decode_workspace_size(&c.d, &n) == c.status);
        // every decode entry point rejects the descriptor the same way, before any launch
        const int b = harness_launches();
        alignas(256) static uint8_t dummy[1024];
        const int32_t* i32 = (const int32_t*)dummy;
        CHECK(mla_decode_partial(&c.d, dummy, dummy, nullptr, i32, i32, 0.1f, dummy, (float*)dummy, dummy,
                                 sizeof dummy, nullptr) == c.status);
        CHECK(mla_decode_plan(&c.d, i32, dummy, sizeof dummy, nullptr) == c.status);
        CHECK(harness_launches() == b);
    }
    CHECK(mla_decode_workspace_size(&base, nullptr) == MLA_ERR_INVALID_ARG);
    CHECK(mla_decode_workspace_size(nullptr, &n) == MLA_ERR_INVALID_ARG);
    // the largest descriptors that are accepted size without overflow
    mla_decode_desc big = desc(1 << 20, 1, 1, 1, 2047);
    CHECK(mla_decode_workspace_size(&big, &n) == MLA_OK && n > ((size_t)1 << 20) * 2 * 4);
    mla_decode_desc wide = desc(1, 16, 65536, 1, (1 << 24) - 1, MLA_BF16, MLA_F32, 1, 0);
    CHECK(mla_decode_workspace_size(&wide, &n) == MLA_OK && n > 0);
}

void merge_cases() {
    harness_clear();
    const int n = 4, rows = 100;
    Buf outs("outs", (size_t)n * rows * 512 * 4), lses("lses", (size_t)n * rows * 4);
    Buf out("out", (size_t)rows * 512 * 4), lse("lse", (size_t)rows * 4);
    int b = harness_launches();
    expect_call(mla_merge_states((float*)outs.p, (float*)lses.p, n, rows, out.p, (float*)lse.p, MLA_F32, nullptr),
                MLA_OK, b, 1);
    b = harness_launches();
    expect_call(mla_merge_states((float*)outs.p, (float*)lses.p, n, rows, out.p, (float*)lse.p, MLA_BF16, nullptr),
                MLA_OK, b, 1);
    b = harness_launches();
    CHECK(mla_merge_states(nullptr, nullptr, n, 0, nullptr, nullptr, MLA_F32, nullptr) == MLA_OK);   // rows 0
    for (int bad_n : {0, -1, 4097})
        CHECK(mla_merge_states((float*)outs.p, (float*)lses.p, bad_n, rows, out.p, (float*)lse.p, MLA_F32,
                               nullptr) == MLA_ERR_INVALID_ARG);
    CHECK(mla_merge_states((float*)outs.p, (float*)lses.p, n, -1, out.p, (float*)lse.p, MLA_F32, nullptr) ==
          MLA_ERR_INVALID_ARG);
    CHECK(mla_merge_states((float*)outs.p, (float*)lses.p, n, rows, out.p, (float*)lse.p, MLA_FP8_E4M3, nullptr) ==
          MLA_ERR_INVALID_ARG);
    CHECK(mla_merge_states(nullptr, (float*)lses.p, n, rows, out.p, (float*)lse.p, MLA_F32, nullptr) ==
          MLA_ERR_INVALID_ARG);
    CHECK(mla_merge_states((float*)(outs.p + 4), (float*)lses.p, n, rows, out.p, (float*)lse.p, MLA_F32,
                           nullptr) == MLA_ERR_INVALID_ARG);
    CHECK(mla_merge_states((float*)outs.p, (float*)(lses.p + 1), n, rows, out.p, (float*)lse.p, MLA_F32,
                           nullptr) == MLA_ERR_INVALID_ARG);
    CHECK(harness_launches() == b);
    harness_clear();
}

void side_kernel_cases() {
    harness_clear();
    // query prep: R 5, H 3, P 128
    {
        const int R = 5, H = 3, P = 128;
        Buf qn("q_nope", (size_t)R * H * P * 2), qp("q_pe", (size_t)R * H * 64 * 2), w("w_uk", (size_t)H * 512 * P * 2);
        Buf qo("q_out", (size_t)R * H * 576 * 2), qs("q_scale", 4);
        mla_query_prep_desc d{R, H, P, MLA_BF16};
        int b = harness_launches();
        expect_call(mla_query_prep(&d, qn.p, qp.p, w.p, nullptr, qo.p, nullptr), MLA_OK, b, 1);
        mla_query_prep_desc d8{R, H, P, MLA_FP8_E4M3};
        b = harness_launches();
        expect_call(mla_query_prep(&d8, qn.p, qp.p, w.p, (float*)qs.p, qo.p, nullptr), MLA_OK, b, 1);
        b = harness_launches();
        CHECK(mla_query_prep(&d8, qn.p, qp.p, w.p, nullptr, qo.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(mla_query_prep(&d, qn.p, qp.p, w.p, (float*)qs.p, qo.p, nullptr) == MLA_ERR_INVALID_ARG);
        for (int p : {0, 8, 17, 272}) {
            mla_query_prep_desc dp{R, H, p, MLA_BF16};
            CHECK(mla_query_prep(&dp, qn.p, qp.p, w.p, nullptr, qo.p, nullptr) != MLA_OK);
        }
        mla_query_prep_desc d0{0, H, P, MLA_BF16};
        CHECK(mla_query_prep(&d0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == MLA_OK);
        CHECK(mla_query_prep(&d, qn.p + 2, qp.p, w.p, nullptr, qo.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(mla_query_prep(nullptr, qn.p, qp.p, w.p, nullptr, qo.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(harness_launches() == b);
    }
    harness_clear();
    // up-projection and the fused merge: R 4, H 2, Vd 128, n 3
    {
        const int R = 4, H = 2, Vd = 128, n = 3;
        Buf ol("o_lat", (size_t)n * R * H * 512 * 4), ls("lses", (size_t)n * R * H * 4), w("w_uv", (size_t)H * Vd * 512 * 2);
        Buf o("out", (size_t)R * H * Vd * 4), lo("lse", (size_t)R * H * 4);
        mla_up_project_desc d{R, H, Vd, MLA_F32, MLA_F32};
        int b = harness_launches();
        expect_call(mla_up_project(&d, ol.p, w.p, o.p, nullptr), MLA_OK, b, 1);
        b = harness_launches();
        expect_call(mla_merge_up_project((float*)ol.p, (float*)ls.p, n, &d, w.p, o.p, (float*)lo.p, nullptr), MLA_OK,
                    b, 1);
        b = harness_launches();
        for (int vd : {0, 16, 33, 544}) {
            mla_up_project_desc dv{R, H, vd, MLA_F32, MLA_F32};
            CHECK(mla_up_project(&dv, ol.p, w.p, o.p, nullptr) != MLA_OK);
        }
        mla_up_project_desc di{R, H, Vd, MLA_FP8_E4M3, MLA_F32};
        CHECK(mla_up_project(&di, ol.p, w.p, o.p, nullptr) == MLA_ERR_INVALID_ARG);
        mla_up_project_desc db{R, H, Vd, MLA_BF16, MLA_F32};
        CHECK(mla_merge_up_project((float*)ol.p, (float*)ls.p, n, &db, w.p, o.p, nullptr, nullptr) ==
              MLA_ERR_INVALID_ARG);
        for (int bad_n : {0, 17})
            CHECK(mla_merge_up_project((float*)ol.p, (float*)ls.p, bad_n, &d, w.p, o.p, nullptr, nullptr) ==
                  MLA_ERR_INVALID_ARG);
        CHECK(mla_up_project(&d, ol.p, w.p + 8, o.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(harness_launches() == b);
    }
    harness_clear();
    // gather: 3 requests, 10 pages of 4 per request, 150 rows
    {
        const int B = 3, pages = 10, maxp = 4;
        const int64_t rows = 150;
        Buf kv("kv", (size_t)pages * 64 * 576 * 2), ks("kv_scale", 4), bt("block_table", (size_t)B * maxp * 4);
        Buf st("seq_starts", (size_t)B * 4), cu("cu_lens", (size_t)(B + 1) * 4), o("out", (size_t)rows * 576 * 2);
        const int32_t* i = (const int32_t*)bt.p;
        int b = harness_launches();
        expect_call(mla_gather_cache(kv.p, MLA_BF16, nullptr, i, B, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p, rows,
                                     o.p, nullptr), MLA_OK, b, 1);
        b = harness_launches();
        expect_call(mla_gather_cache(kv.p, MLA_FP8_E4M3, (float*)ks.p, i, B, pages, maxp, (int32_t*)st.p,
                                     (int32_t*)cu.p, rows, o.p, nullptr), MLA_OK, b, 1);
        b = harness_launches();
        CHECK(mla_gather_cache(kv.p, MLA_FP8_E4M3, nullptr, i, B, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p, rows,
                               o.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(mla_gather_cache(kv.p, MLA_F32, nullptr, i, B, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p, rows, o.p,
                               nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(mla_gather_cache(kv.p, MLA_BF16, nullptr, i, B, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p,
                               ((int64_t)1 << 34) + 1, o.p, nullptr) == MLA_ERR_UNSUPPORTED);
        CHECK(mla_gather_cache(kv.p, MLA_BF16, nullptr, i, B, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p, 0, nullptr,
                               nullptr) == MLA_OK);
        CHECK(mla_gather_cache(kv.p, MLA_BF16, nullptr, i, 0, pages, maxp, (int32_t*)st.p, (int32_t*)cu.p, rows, o.p,
                               nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(harness_launches() == b);
    }
    harness_clear();
    // two-way merge: 37 rows of 128
    {
        const int rows = 37, hd = 128;
        Buf po("prefix_out", (size_t)rows * hd * 4), pl("prefix_lse", (size_t)rows * 4);
        Buf so("suffix_out", (size_t)rows * hd * 4), sl("suffix_lse", (size_t)rows * 4);
        Buf o("out", (size_t)rows * hd * 4), l("lse", (size_t)rows * 4);
        int b = harness_launches();
        expect_call(mla_merge_two_states(rows, hd, MLA_F32, MLA_BF16, po.p, (float*)pl.p, so.p, (float*)sl.p, o.p,
                                         (float*)l.p, nullptr), MLA_OK, b, 1);
        b = harness_launches();
        for (int h : {0, 2, 6, 4100})
            CHECK(mla_merge_two_states(rows, h, MLA_F32, MLA_F32, po.p, (float*)pl.p, so.p, (float*)sl.p, o.p,
                                       (float*)l.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(mla_merge_two_states(0, hd, MLA_F32, MLA_F32, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr) == MLA_OK);
        CHECK(mla_merge_two_states(rows, hd, MLA_F32, MLA_F32, po.p + 4, (float*)pl.p, so.p, (float*)sl.p, o.p,
                                   (float*)l.p, nullptr) == MLA_ERR_INVALID_ARG);
        CHECK(harness_launches() == b);
    }
    harness_clear();
    for (int s : {0, -1, -2, -3, -4, -5, -6, 1, 12345}) CHECK(mla_status_string(s) != nullptr);
}

}  // namespace

// A caller that claims more workspace than it has: the layer cannot see the
// buffer's size, so the call goes through, and the stand-ins must flag the
// split partials' extent (the run is then expected to fail).
int planted_short_workspace() {
    DecodeArgs a(desc(64, 1, 128, 4096, 64));
    harness_clear();
    Buf q("q", a.q->n), kv("kv", a.kv->n), bt("block_table", a.bt->n), sl("seq_lens", a.sl->n);
    Buf out("out", a.out->n), lse("lse", a.lse->n), ws("workspace", a.ws_bytes - 4096);
    const int st = mla_decode_partial(&a.d, q.p, kv.p, nullptr, (const int32_t*)bt.p, (const int32_t*)sl.p, 0.1f,
                                      out.p, (float*)lse.p, ws.p, a.ws_bytes, nullptr);
    printf("planted short workspace: status %d, %d extent failures\n", st, harness_failures());
    return harness_failures() > 0 ? 1 : 0;
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "--plant-short-workspace") == 0) return planted_short_workspace();
    decode_cases();
    noalloc_cases();
    descriptor_cases();
    merge_cases();
    side_kernel_cases();
    const int stub_failures = harness_failures();
    printf("boundary driver: %d launches checked, %d check failures, %d extent failures\n", harness_launches(),
           g_fails, stub_failures);
    return g_fails == 0 && stub_failures == 0 ? 0 : 1;
}
