/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) absorbed-MQA MLA decode library.
 *
 * What the library computes
 * -------------------------
 * Multi-head Latent Attention decode in its absorbed-MQA form: the KV cache is
 * ONE latent head of 576 values per token (kv_c 512 + k_pe 64), and the query
 * has been absorbed into that latent space (512 + 64 = 576 per head), so no
 * per-head K/V is ever expanded (page 4, "MLA Prefill vs Decode", the
 * Prefill/Decode table and the two paragraphs under it; page 1, "实现拆解"
 * item 5, the W_UK_T matmul).  For every query row r = (request b, query
 * token t, head h) and the n visible cache tokens j of this shard:
 *     s_j   = scale * kv_scale * <q_r, k_j>            (all 576 dims)
 *     lse_r = ln sum_j exp(s_j)                         (natural log)
 *     o_r   = kv_scale * sum_j exp(s_j - lse_r) * k_j[0:512]
 * The decode returns BOTH o and lse (page 2, the forward_mqa line of the
 * forward_impl excerpt), because under Decode Context Parallelism each rank
 * holds a sequence shard of the cache, computes partial attention over it,
 * and the partials are merged with LSE weights (page 4, "什么是 DCP" and
 * "DCP 在 Prefill 与 Decode 中的不同角色").  The merge is the elementwise LSE
 * rescaling of merge_attn_states (page 4, "Chunked Prefill 与 LSE Merge").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument named as device memory must point to memory the
 *    current HIP device can access; the CALLER owns all buffers, including the
 *    workspace.  The library allocates and frees nothing in these calls and
 *    keeps no per-call state, so calls on different streams do not interfere
 *    (two calls sharing one workspace must not overlap in time).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work: it never synchronises the host.  Results
 *    are valid once the stream has reached the call.
 *  - Host-checkable argument errors are reported by the return value BEFORE
 *    any device work is enqueued (see mla_status).  A failed kernel launch
 *    returns MLA_ERR_HIP.  Contract violations that only the device can see
 *    never make a kernel access memory outside its arguments, but give
 *    meaningless results for the rows concerned: a seq_len beyond
 *    max_pages_per_seq * page_size (or below 0) is clamped into
 *    [0, max_pages_per_seq * page_size]; a live block-table entry outside
 *    [0, num_pages) is clamped into the pool (a negative or too large id
 *    reads page num_pages - 1).
 *  - Layouts are dense, row-major, with no padding unless stated.  Query and
 *    output rows of a request are ordered (query token t, head h).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
    MLA_BF16 = 0,      /* bfloat16 */
    MLA_FP8_E4M3 = 1,  /* OCP FP8 E4M3 ("e4m3fn"), the gfx950 native fp8 */
    MLA_F32 = 2        /* IEEE binary32 */
} mla_dtype;

/* Return codes. */
typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or shape */
    MLA_ERR_UNSUPPORTED = -2,  /* valid but not supported combination */
    MLA_ERR_WORKSPACE = -3,    /* workspace missing or too small */
    MLA_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
    MLA_ERR_SCRATCH_LIMIT = -5 /* mla_decode_partial_noalloc: the descriptor needs more
                                  workspace than the static scratch holds */
} mla_status;

/* Fixed model dimensions of the latent cache (page 4: 512 + 64 = 576). */
#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_QK_DIM 576
/* The only supported page size (tokens per cache page). */
#define MLA_PAGE_SIZE 64

/* Shape and type descriptor of one decode call (one DCP shard).
 * The decode schedule is sized by q_len * num_heads rows per request, with ONE
 * KV head; under DCP the gathered or replicated query carries num_heads already
 * multiplied by the DCP world size (page 2, "实现拆解" item 2 and the
 * FlashMLA _build_decode excerpt). */
typedef struct mla_decode_desc {
    int32_t batch;              /* B >= 1 requests */
    int32_t q_len;              /* query tokens per request, 1 .. 16 */
    int32_t num_heads;          /* H >= 1 query heads (x DCP world size if gathered) */
    int32_t page_size;          /* must be MLA_PAGE_SIZE */
    int32_t num_pages;          /* pages in the cache pool, >= 1 */
    int32_t max_pages_per_seq;  /* row stride of block_table, >= 1 */
    int32_t kv_dtype;           /* MLA_BF16 or MLA_FP8_E4M3; q has the same dtype */
    int32_t out_dtype;          /* MLA_F32 or MLA_BF16 for `out` */
    int32_t causal;             /* q_len > 1 only: 1 = query token t sees the first
                                   seq_len - (q_len - 1 - t) tokens; 0 = all tokens */
    int32_t num_splits;         /* 0 = automatic split-KV; k > 0 = exactly
                                   min(k, pages of the request) splits per request */
} mla_decode_desc;

/* Bytes of device workspace mla_decode_partial needs for `desc`.
 * Depends only on the descriptor (never on seq_lens), so a caller can size it
 * once.  Returns MLA_OK, or MLA_ERR_INVALID_ARG / MLA_ERR_UNSUPPORTED for a bad
 * descriptor.  No device access. */
int mla_decode_workspace_size(const mla_decode_desc* desc, size_t* bytes);

/* Absorbed-MQA decode of one KV shard: partial output + LSE per query row.
 * (page 4, "MLA Prefill vs Decode"; page 2, the forward_mqa call that returns
 *  attn_out and lse; page 2 FlashMLA excerpt for the per-step split metadata
 *  built from seq_lens and q_len x heads with one KV head.)
 *
 *   q           device, [B][q_len][H][576] of kv_dtype (bf16, or e4m3 codes);
 *               16-byte aligned.  For fp8 the caller folds its per-tensor query
 *               scale into `scale`.
 *   kv_cache    device, [num_pages][64][576] of kv_dtype, 16-byte aligned.
 *               Token j of request b is row j % 64 of page block_table[b][j / 64].
 *               Cache rows past seq_len and unused pages are never used.
 *   kv_scale    device float[1]: the per-tensor cache scale for MLA_FP8_E4M3
 *               (required); must be NULL for MLA_BF16.
 *   block_table device int32 [B][max_pages_per_seq]; entries at or beyond
 *               ceil(seq_len / 64) are never read (may be -1).
 *   seq_lens    device int32 [B]: cache tokens per request in this shard,
 *               including the q_len new ones; 0 is allowed (empty shard).
 *   scale       softmax scale applied to q.k (e.g. 1/sqrt(192)); finite and > 0.
 *   out         device, [B][q_len][H][512] of out_dtype, 16-byte aligned.
 *   lse         device float [B][q_len][H]: natural-log LSE of the scaled
 *               logits; -inf (and out = 0) for a row that sees no token.
 *   workspace   device, >= mla_decode_workspace_size() bytes, 256-byte aligned.
 * Work: a planning kernel reads seq_lens on the device and writes the split
 * list into the workspace; the split-KV decode kernel streams the pages; a
 * combine kernel LSE-merges the splits of each row into `out` / `lse`.  A
 * request decoded in one piece is written straight to out in fp32 or bf16;
 * one cut into several pieces passes through bf16 partial outputs (each
 * normalised, so rounded within 2^-9 of its magnitude) and fp32 partial LSEs.
 * Returns MLA_OK or a negative mla_status (before any device work on a bad
 * argument). */
int mla_decode_partial(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                       const float* kv_scale, const int32_t* block_table,
                       const int32_t* seq_lens, float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's static device scratch on each GPU (the workspace of
 * mla_decode_partial_noalloc). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* mla_decode_partial for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same decode, with the library's own static device scratch
 * in place of a caller workspace.  Arguments, results, validation and errors
 * are those of mla_decode_partial, minus the workspace.
 *  - The scratch is a file-scope device array of MLA_NOALLOC_SCRATCH_BYTES
 *    (128 MiB), one per GPU the library runs on, held from library load until
 *    the process ends.  Its address on the current device is looked up on the
 *    first call on that device (make that first call outside graph capture).
 *  - A descriptor whose workspace (mla_decode_workspace_size) exceeds the
 *    scratch returns MLA_ERR_SCRATCH_LIMIT before any device work.  The
 *    workspace holds 131,616 bytes per work unit (bf16 split partials), and
 *    the automatic split of B requests of T 128-row tiles sizes for
 *    ceil((256 / T + B) / 8) * 8 * T units: up to 1,016 units fit (for
 *    example B = 760 with 128 heads, or B = 128 with 512 heads); 256 fixed
 *    splits of a long sequence do not.
 *  - The call allocates and frees nothing: no hipMalloc or hipFree and no
 *    allocating library routine.
 *  - Every call on a GPU shares that GPU's scratch, which keeps the last
 *    call's contents; nothing in it needs to start at zero (each call writes
 *    its split plan before reading it).  Calls that overlap in time on one GPU
 *    (on different streams, or from threads without ordering) race on the
 *    scratch and give wrong results: order them on one stream. */
int mla_decode_partial_noalloc(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                               const float* kv_scale, const int32_t* block_table,
                               const int32_t* seq_lens, float scale, void* out, float* lse,
                               void* stream);

/* The split plan of a decode step alone, for reuse by every layer's decode of
 * that step (page 2, the flashmla.py _build_decode excerpt: the scheduler
 * metadata comes from seq_lens and q tokens x heads in the backend's per-step
 * metadata build, apart from the attention calls that consume it).
 *   desc, seq_lens, workspace: as for mla_decode_partial.
 * Enqueues one planner kernel on `stream` that writes the per-request split
 * counts and the work list into the workspace; nothing else of the workspace
 * is touched.  Returns MLA_OK or a negative mla_status (before any device work
 * on a bad argument). */
int mla_decode_plan(const mla_decode_desc* desc, const int32_t* seq_lens, void* workspace,
                    size_t workspace_bytes, void* stream);

/* mla_decode_partial without the planning step: the split-KV decode and the
 * combine follow the plan that mla_decode_plan left in `workspace`.  Arguments
 * and results are those of mla_decode_partial.  The workspace must hold the
 * plan for the same descriptor and the same seq_lens values, made earlier in
 * stream order; the plan stays valid across calls (each call only rewrites
 * the split partials), so the calls of one step on one workspace must not
 * overlap.  A work item or split count that does not fit the descriptor is
 * skipped rather than followed (its rows are then not written); a plan for
 * other seq_lens gives wrong results but no access outside the arguments. */
int mla_decode_partial_planned(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                               const float* kv_scale, const int32_t* block_table,
                               const int32_t* seq_lens, float scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* LSE merge of n partial results per row (page 4, "Chunked Prefill 与 LSE
 * Merge": merge_attn_states' elementwise LSE rescaling; "DCP 在 Prefill 与
 * Decode 中的不同角色": DCP decode merges per-rank partials with LSE weights).
 *   outs   device float [n][rows][512], 16-byte aligned (partial i at outs + i*rows*512)
 *   lses   device float [n][rows] (natural log; -inf marks an empty partial)
 *   out    device [rows][512] of out_dtype (MLA_F32 or MLA_BF16), 16-byte aligned
 *   lse    device float [rows]
 * Per row: lse = ln sum_i exp(lse_i); out = sum_i exp(lse_i - lse) * outs_i;
 * a row whose inputs are all empty gets out = 0, lse = -inf.
 * n in 1 .. 4096, rows >= 0.  out/lse must not overlap the inputs. */
int mla_merge_states(const float* outs, const float* lses, int32_t n, int32_t rows,
                     void* out, float* lse, int32_t out_dtype, void* stream);

/* Shape and type descriptor of a query preparation. */
typedef struct mla_query_prep_desc {
    int32_t rows;       /* query rows R >= 0 (requests x query tokens) */
    int32_t num_heads;  /* H >= 1 */
    int32_t nope_dim;   /* P: per-head no-rope query width, a multiple of 16 in 16 .. 256 */
    int32_t out_dtype;  /* MLA_BF16 or MLA_FP8_E4M3 */
} mla_query_prep_desc;

/* Prepare the decode query: absorb each head's no-rope part into the latent
 * space through W_UK_T and join the rope part (page 1, "实现拆解" item 5, the
 * W_UK_T batched matmul; page 4, "MLA Prefill vs Decode", the query absorbed
 * into the latent space; page 2, the decode section of the forward_impl
 * excerpt: nope and pe concatenated, or concatenated and quantised to fp8
 * with a per-tensor query scale).  For every row r and head h:
 *     q_out[r][h][0:512]   = sum_p q_nope[r][h][p] * W_UK_T[h][p][0:512]   (fp32 sums)
 *     q_out[r][h][512:576] = q_pe[r][h][0:64]
 * stored as bf16 (round to nearest even), or for MLA_FP8_E4M3 as the e4m3
 * code of value / q_scale (fp32 division; round to nearest even, saturating
 * at +-448).  The result is the `q` mla_decode_partial takes; with fp8 the
 * caller folds q_scale into the decode's `scale`.
 *   q_nope   device bf16 [R][H][P], 16-byte aligned
 *   q_pe     device bf16 [R][H][64], 16-byte aligned
 *   w_uk     device bf16 [H][512][P], 16-byte aligned: w_uk[h][l][p] =
 *            W_UK_T[h][p][l] (the weights stored latent-major, a one-time
 *            permutation at weight load)
 *   q_scale  device float[1], required for MLA_FP8_E4M3 (finite, > 0), NULL for bf16
 *   q_out    device [R][H][576] of out_dtype, 16-byte aligned; must not
 *            overlap the inputs
 * R = 0 enqueues nothing.  Returns MLA_OK or a negative mla_status before any
 * device work on a bad argument. */
int mla_query_prep(const mla_query_prep_desc* desc, const void* q_nope, const void* q_pe,
                   const void* w_uk, const float* q_scale, void* q_out, void* stream);

/* Shape and type descriptor of an output up-projection. */
typedef struct mla_up_project_desc {
    int32_t rows;        /* R >= 0 (requests x query tokens) */
    int32_t num_heads;   /* H >= 1 */
    int32_t v_head_dim;  /* Vd: per-head value width, a multiple of 32 in 32 .. 512 */
    int32_t in_dtype;    /* MLA_F32 or MLA_BF16: the latent output's type */
    int32_t out_dtype;   /* MLA_F32 or MLA_BF16 */
} mla_up_project_desc;

/* Map each head's 512-dim latent attention output into its value space
 * through W_UV (page 1, "关键源码片段": the attention output is
 * num_heads x v_head_dim per token; page 4, "MLA Prefill vs Decode": W_UV
 * decompresses the latent into per-head values):
 *     out[r][h][v] = sum_l W_UV[h][v][l] * o_lat[r][h][l]
 * with fp32 sums; an fp32 o_lat enters the bf16 matrix cores as two bf16
 * terms (x = hi + lo to within 2^-17 |x|), so the result keeps near-fp32
 * accuracy; a bf16 output is rounded to nearest even.
 *   o_lat  device [R][H][512] of in_dtype, 16-byte aligned (mla_decode_partial's
 *          or mla_merge_states' out)
 *   w_uv   device bf16 [H][Vd][512], 16-byte aligned (row v of head h: the
 *          512 latent weights of value dim v)
 *   out    device [R][H][Vd] of out_dtype, 16-byte aligned; must not overlap
 *          the inputs
 * R = 0 enqueues nothing.  Returns MLA_OK or a negative mla_status before any
 * device work on a bad argument. */
int mla_up_project(const mla_up_project_desc* desc, const void* o_lat, const void* w_uv,
                   void* out, void* stream);

/* mla_merge_states fused in front of mla_up_project: the latent input of row
 * (r, h) is the LSE merge of n fp32 partials (DCP shard results; page 4, "DCP
 * 在 Prefill 与 Decode 中的不同角色": per-rank partials merged with LSE
 * weights), and is mapped through W_UV without going through memory:
 *     o_lat = sum_i exp(lse_i - lse) * outs_i,  lse = ln sum_i exp(lse_i),
 *     out[r][h][v] = sum_l W_UV[h][v][l] * o_lat[l]
 *   outs   device float [n][R * H][512], 16-byte aligned (rows ordered (r, h))
 *   lses   device float [n][R * H]; -inf marks an empty partial (never read)
 *   desc   as for mla_up_project, with in_dtype = MLA_F32
 *   out    device [R][H][Vd] of desc->out_dtype, 16-byte aligned
 *   lse    device float [R * H] receives the merged LSE, or NULL
 * n in 1 .. 16.  A row whose partials are all empty gets out = 0, lse = -inf. */
int mla_merge_up_project(const float* outs, const float* lses, int32_t n,
                         const mla_up_project_desc* desc, const void* w_uv, void* out, float* lse,
                         void* stream);

/* Gather the latent cache rows of each request's context chunk into one
 * contiguous bf16 buffer, dequantising an e4m3 cache (page 4, "与非 DCP 的流程对比":
 * each prefill chunk's context is taken out of the paged cache by
 * gather_and_maybe_dequant_cache; page 2, "实现拆解" items 3 and 4: the
 * gather whose requests start at seq_starts).  Output row cu_lens[b] + i is
 * token seq_starts[b] + i of request b (row t % 64 of page
 * block_table[b][t / 64]), for i < cu_lens[b + 1] - cu_lens[b]:
 *   bf16 cache:  copied;
 *   e4m3 cache:  bf16(fp32(value) * kv_scale), the fp32 product rounded to
 *                nearest even.
 *   kv_cache     device [num_pages][64][576] of kv_dtype, 16-byte aligned
 *   kv_scale     device float[1] for MLA_FP8_E4M3 (NULL for MLA_BF16)
 *   block_table  device int32 [batch][max_pages_per_seq]
 *   seq_starts   device int32 [batch], >= 0
 *   cu_lens      device int32 [batch + 1], non-decreasing, cu_lens[0] = 0
 *   total_rows   rows to write (normally cu_lens[batch], which the host passes
 *                because it sizes the launch); rows past cu_lens[batch] are zeros
 *   out          device bf16 [total_rows][576], 16-byte aligned
 * A row whose token lies past the block table or whose page id is outside
 * [0, num_pages) is written as zeros. */
int mla_gather_cache(const void* kv_cache, int32_t kv_dtype, const float* kv_scale,
                     const int32_t* block_table, int32_t batch, int32_t num_pages,
                     int32_t max_pages_per_seq, const int32_t* seq_starts, const int32_t* cu_lens,
                     int64_t total_rows, void* out, void* stream);

/* merge_attn_states of a prefix and a suffix partial result (page 4,
 * "Chunked Prefill 与 LSE Merge"): per row, with w_i = exp(lse_i - max),
 *   out = (w_p prefix + w_s suffix) / (w_p + w_s),  lse = max + ln(w_p + w_s);
 * a -inf LSE marks an empty partial; two empty inputs give out = 0, lse = -inf.
 * LSE values must be finite or -inf.
 *   prefix_out, suffix_out  device [rows][head_dim] of in_dtype (MLA_F32 or MLA_BF16)
 *   prefix_lse, suffix_lse  device float [rows]
 *   out                     device [rows][head_dim] of out_dtype (MLA_F32 or MLA_BF16)
 *   lse                     device float [rows], or NULL when not wanted
 * head_dim: a multiple of 4 in 4 .. 4096; every pointer 16-byte aligned.  out
 * may not overlap the inputs. */
int mla_merge_two_states(int32_t rows, int32_t head_dim, int32_t in_dtype, int32_t out_dtype,
                         const void* prefix_out, const float* prefix_lse, const void* suffix_out,
                         const float* suffix_lse, void* out, float* lse, void* stream);

/* Human-readable text of a status code (static storage; never NULL). */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
