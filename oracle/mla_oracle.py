"""Plain fp64 CPU oracle for absorbed-MQA MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``mla_latent_decode_absorbed_amd``) never does, and this module imports nothing
from it: the two share no code.

What is computed, and where the pages say so
--------------------------------------------
* Decode keeps the KV cache as ONE latent head of 576 values per token
  (kv_c 512 + k_pe 64) and absorbs the query into that latent space, so the
  query is also 576 wide per head (page 4, "MLA Prefill vs Decode" table and the
  paragraph under it; the 512 + 64 = 576 figure is in page 4's
  "AllGather latent KV" table).  The query absorption itself (q_nope through
  W_UK) is the "W_UK_T" batched matmul of page 1, "实现拆解" item 5.
* The decode call returns BOTH the attention output and its log-sum-exp
  (page 2, the ``forward_mqa`` line of the ``forward_impl`` excerpt; page 1,
  "风险与影响" item 2, "DCP decode-LSE").
* Partial results over disjoint KV sets are combined by LSE rescaling
  (``merge_attn_states``: page 4, "Chunked Prefill 与 LSE Merge"); under DCP,
  each rank computes partial attention over its KV shard and the partials are
  merged with LSE weights (page 4, "DCP 在 Prefill 与 Decode 中的不同角色").
* DCP shards the KV cache along the sequence, each rank holding 1/D of it
  (page 4, "什么是 DCP").

Each function below is the plain mathematical definition written out, in fp64,
on the exact input values (bf16 and OCP e4m3 codes are decoded exactly).  Library
primitives used as steps: numpy matmul, exp, log, max, fancy indexing.

Readings where the pages are silent (each is listed in the design doc):
* scale is an argument (the configs use 1/sqrt(192)); the LSE is the NATURAL log
  of sum_j exp(s_j) over the SCALED logits s_j = scale * kv_scale * <q, k_j>;
* partial outputs are normalised (weights sum to one); the merge weight of
  partial i is exp(lse_i - lse);
* V is cache dims [0, 512) of the same rows; the output is the 512-dim latent;
* with q_len > 1 and causal, query token t (0-based) sees the first
  n - (q_len - 1 - t) cache tokens (seq_len n includes the new tokens);
* a row that sees no token has o = 0 and lse = -inf; the merge ignores such
  inputs, and an all-empty merge gives o = 0, lse = -inf;
* fp8: the cache holds OCP e4m3fn codes times a per-tensor kv_scale; logits are
  scale * kv_scale * (q_hat . k_hat) with any query scale folded into ``scale``
  by the caller; the output is kv_scale * sum_j w_j v_hat_j.
"""
from __future__ import annotations

import numpy as np

#: latent (kv_c) width, rope (k_pe) width and their sum (page 4, per-token
#: communication table: kv_lora_rank + rope_dim = 512 + 64 = 576).
LATENT_DIM = 512
ROPE_DIM = 64
QK_DIM = LATENT_DIM + ROPE_DIM
#: tokens per cache page (the pages do not fix it; the workloads use 64).
PAGE_SIZE = 64


# --------------------------------------------------------------------------
# exact decoding of stored values
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16 / int16) -> float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32, so shifting the pattern
    into the high 16 bits of a uint32 and reinterpreting gives the same value.
    """
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_bits_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("e4m3fn") codes (uint8) -> float64, by the format's formula.

    sign = bit 7, exponent E = bits 6..3 (bias 7), mantissa m = bits 2..0.
    E == 0: (-1)^s * m * 2^-9 (subnormal); otherwise (-1)^s * (1 + m/8) * 2^(E-7).
    E == 15 with m == 7 is NaN; there are no infinities; max finite is 448.
    """
    c = np.asarray(codes).view(np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * m.astype(np.float64) * 2.0 ** -9
    nrm = sign * (1.0 + m.astype(np.float64) / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    out = np.where(e == 0, sub, nrm)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out


# --------------------------------------------------------------------------
# paged cache addressing
# --------------------------------------------------------------------------
def gather_request_rows(kv_cache: np.ndarray, block_row: np.ndarray, n: int,
                        page_size: int = PAGE_SIZE) -> np.ndarray:
    """Logical token rows 0..n-1 of one request from a paged cache.

    Token j lives in physical page ``block_row[j // page_size]`` at slot
    ``j % page_size`` (the per-request block table of page 4, "Prefill 阶段的
    DCP 设计", step 1).  Only pages holding tokens < n are dereferenced.
    """
    if n <= 0:
        return np.zeros((0, kv_cache.shape[-1]), dtype=np.float64)
    j = np.arange(n)
    pages = np.asarray(block_row)[j // page_size]
    return kv_cache[pages, j % page_size, :]


def visible_lengths(n: int, q_len: int, causal: bool) -> np.ndarray:
    """Number of cache tokens each query token t = 0..q_len-1 attends to.

    Non-causal: all n.  Causal (bottom-right aligned, the n cache tokens
    include the q_len new ones): token t sees n - (q_len - 1 - t).
    """
    t = np.arange(q_len)
    if causal:
        return np.maximum(n - (q_len - 1 - t), 0)
    return np.full(q_len, max(n, 0))


# --------------------------------------------------------------------------
# the attention definition
# --------------------------------------------------------------------------
def attend_rows(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                scale: float, kv_scale: float = 1.0):
    """softmax attention of some query rows over the SAME visible key rows.

    q_rows [R][576], k_rows [n][576], v_rows [n][512] (all float64).
    s_j = scale * kv_scale * <q, k_j>;  mu = max_j s_j;  w_j = exp(s_j - mu);
    l = sum_j w_j;  lse = mu + ln l;  o = kv_scale * sum_j (w_j / l) v_j.
    n == 0 gives o = 0 and lse = -inf.
    """
    R = q_rows.shape[0]
    if k_rows.shape[0] == 0:
        return np.zeros((R, v_rows.shape[-1])), np.full(R, -np.inf)
    s = (scale * kv_scale) * (q_rows @ k_rows.T)          # [R][n]
    mu = s.max(axis=1, keepdims=True)
    w = np.exp(s - mu)
    l = w.sum(axis=1, keepdims=True)
    lse = (mu + np.log(l))[:, 0]
    o = kv_scale * ((w / l) @ v_rows)
    return o, lse


def decode_partial_ref(q: np.ndarray, kv_cache: np.ndarray, block_table: np.ndarray,
                       seq_lens: np.ndarray, scale: float, kv_scale: float = 1.0,
                       causal: bool | None = None, requests=None):
    """Absorbed-MQA decode of one KV shard: out [B][q_len][H][512], lse [B][q_len][H].

    q [B][q_len][H][576] float64 (already absorbed; rope applied);
    kv_cache [P][page][576] float64 (one latent head per token);
    block_table [B][max_pages] int; seq_lens [B] int.
    K_b = the request's logical rows (all 576 dims), V_b = K_b[:, :512].
    ``causal`` defaults to (q_len > 1).  ``requests`` restricts the work to a
    subset of request indices (others are left as NaN) for sampled checks.
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len, H, D = q.shape
    assert D == QK_DIM and kv_cache.shape[-1] == QK_DIM
    if causal is None:
        causal = q_len > 1
    page = kv_cache.shape[1]
    out = np.full((B, q_len, H, LATENT_DIM), np.nan)
    lse = np.full((B, q_len, H), np.nan)
    todo = range(B) if requests is None else requests
    for b in todo:
        n = int(seq_lens[b])
        k_all = gather_request_rows(kv_cache, block_table[b], n, page)
        for t, n_t in enumerate(visible_lengths(n, q_len, causal)):
            k_rows = k_all[:n_t]
            o, l = attend_rows(q[b, t], k_rows, k_rows[:, :LATENT_DIM], scale, kv_scale)
            out[b, t] = o
            lse[b, t] = l
    return out, lse


def merge_ref(outs: np.ndarray, lses: np.ndarray):
    """LSE merge of n partial results per row: ``merge_attn_states`` generalised.

    outs [n][R][V], lses [n][R].  Per row: mu = max_i lse_i; if mu = -inf the
    row is empty (o = 0, lse = -inf); otherwise a_i = exp(lse_i - mu) (zero for
    -inf inputs), S = sum_i a_i, lse = mu + ln S, o = sum_i (a_i / S) o_i.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    mu = lses.max(axis=0)                                   # [R]
    empty = np.isneginf(mu)
    mu_safe = np.where(empty, 0.0, mu)
    a = np.where(np.isneginf(lses), 0.0, np.exp(lses - mu_safe[None, :]))   # [n][R]
    S = a.sum(axis=0)
    S_safe = np.where(empty, 1.0, S)
    lse = np.where(empty, -np.inf, mu_safe + np.log(S_safe))
    # an input with weight 0 contributes nothing, even if its output is garbage
    contrib = np.where((a > 0)[:, :, None], (a / S_safe[None, :])[:, :, None] * outs, 0.0)
    o = np.where(empty[:, None], 0.0, contrib.sum(axis=0))
    return o, lse


# --------------------------------------------------------------------------
# DCP sequence sharding (t mod D)
# --------------------------------------------------------------------------
def dcp_shard_len(n: int, D: int, r: int) -> int:
    """Tokens of a length-n sequence held by shard r of D under t -> t mod D."""
    return max(0, (n - r + D - 1) // D)


def dcp_shard_positions(n: int, D: int, r: int) -> np.ndarray:
    """Global positions of shard r's local tokens, in increasing order (local j <-> j*D + r)."""
    return np.arange(r, n, D)


# --------------------------------------------------------------------------
# the non-absorbed (decompressed) form, used only to pin the absorbed one
# --------------------------------------------------------------------------
def absorb_query(q_nope: np.ndarray, q_pe: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """Absorbed query of page 1's W_UK_T matmul: q_lat[h] = W_UK[h]^T q_nope[h], then concat q_pe.

    q_nope [H][P], q_pe [H][R], w_uk [H][P][512] (W_UK[h] maps a 512-dim latent to
    head h's P-dim key) -> [H][512 + R].
    """
    q_lat = np.einsum('hp,hpl->hl', q_nope, w_uk)
    return np.concatenate([q_lat, q_pe], axis=-1)


def mha_unabsorbed_ref(q_nope, q_pe, kv_c, k_pe, w_uk, w_uv, scale):
    """Standard multi-head attention after decompressing the latent cache (page 4,
    "MLA Prefill vs Decode": kv_c through W_UK/W_UV into per-head K/V).

    q_nope [H][P], q_pe [H][R], kv_c [n][512], k_pe [n][R], w_uk [H][P][512],
    w_uv [H][Vd][512].  Head h: K_h[j] = [W_UK[h] kv_c[j], k_pe[j]] (P + R dims),
    V_h[j] = W_UV[h] kv_c[j]; scores scale * <[q_nope[h], q_pe[h]], K_h[j]>.
    Returns out [H][Vd], lse [H], and the raw scores [H][n].
    """
    H = q_nope.shape[0]
    n = kv_c.shape[0]
    outs, lses, scores = [], [], []
    for h in range(H):
        k_h = np.concatenate([kv_c @ w_uk[h].T, k_pe], axis=1)      # [n][P+R]
        v_h = kv_c @ w_uv[h].T                                      # [n][Vd]
        q_h = np.concatenate([q_nope[h], q_pe[h]])                  # [P+R]
        s = scale * (k_h @ q_h)                                     # [n]
        mu = s.max()
        w = np.exp(s - mu)
        l = w.sum()
        outs.append((w / l) @ v_h)
        lses.append(mu + np.log(l))
        scores.append(s)
    return np.stack(outs), np.array(lses), np.stack(scores).reshape(H, n)


# --------------------------------------------------------------------------
# query preparation: absorption, concatenation and quantisation of the query
# --------------------------------------------------------------------------
# The decode path consumes the absorbed query: head h's no-rope part is mapped
# into the latent space by the per-head W_UK_T batched matmul (page 1,
# "实现拆解" item 5; page 4, "MLA Prefill vs Decode", the query absorbed by an
# einsum into the latent space), then joined with the rope part, either as a
# plain concatenation or as a concatenation quantised to fp8 with a per-tensor
# query scale (page 2, the ``forward_impl`` decode excerpt:
# ``_decode_concat_quant_fp8_op(mqa_ql_nope, mqa_q_pe, self._q_scale)``).
def query_prep_ref(q_nope: np.ndarray, q_pe: np.ndarray, w_uk_lp: np.ndarray) -> np.ndarray:
    """Exact absorbed query rows: [R][H][512 + 64] in fp64.

    q_nope [R][H][P], q_pe [R][H][64], w_uk_lp [H][512][P], where w_uk_lp[h][l][p]
    is W_UK_T[h][p][l] (the weights stored latent-major).  Each (row, head) is
    ``absorb_query`` of that row: q_lat[l] = sum_p q_nope[p] W_UK_T[h][p][l].
    """
    R, H, _ = q_nope.shape
    w_uk = np.transpose(w_uk_lp, (0, 2, 1))            # [H][P][512]
    return np.stack([absorb_query(q_nope[r], q_pe[r], w_uk) for r in range(R)])


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    A finite bf16 has 8 significant bits: values in [2^e, 2^(e+1)) are spaced
    2^(e-7), down to the subnormal spacing 2^-133 below 2^-126.  Values past the
    largest finite bf16 (by half a spacing or more) round to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, -126.0) - 7.0)
    q = np.rint(a / spacing) * spacing                  # rint: ties to even
    q = np.where(q >= 2.0 ** 128, np.inf, q)
    q = np.where(np.isnan(x), np.nan, q)
    v = np.where(np.signbit(x), -q, q).astype(np.float32)   # exact: q is a bf16 value
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


#: largest finite OCP e4m3 magnitude, 1.75 * 2^8
E4M3_MAX = 448.0


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> OCP FP8 E4M3 codes (uint8), round to nearest, ties to even,
    saturating: magnitudes above 448 give +-448 (a quantiser with a fixed scale
    clamps to the format's range; the format has no infinities).

    Normal values in [2^e, 2^(e+1)), e >= -6, have 4 significant bits (spacing
    2^(e-3)); below 2^-6 the subnormal spacing is 2^-9.  NaN gives 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    # magnitudes of 1024 and more (and infinities) saturate like 1024; NaN is
    # set aside and coded at the end
    a = np.where(np.isnan(x), 0.0, np.minimum(np.abs(x), 1024.0))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, -6.0) - 3.0)
    q = np.minimum(np.rint(a / spacing) * spacing, E4M3_MAX)
    ee = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    E = np.where(normal, ee + 7.0, 0.0)
    M = np.where(normal, (q / np.exp2(ee) - 1.0) * 8.0, q / 2.0 ** -9)
    code = (E.astype(np.int64) << 3) | np.rint(M).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def query_prep_codes(q_exact: np.ndarray, out_dtype: str, q_scale: float = 1.0) -> np.ndarray:
    """Encode exact query values as the prepared query's storage: bf16 bit
    patterns, or e4m3 codes of the value divided by the per-tensor q_scale
    (the division taken in fp32, as the stored scale is an fp32 number)."""
    if out_dtype == "bf16":
        return bf16_encode(q_exact)
    if out_dtype == "fp8":
        return e4m3_encode(np.float32(q_exact) / np.float32(q_scale))
    raise ValueError(out_dtype)


# --------------------------------------------------------------------------
# output up-projection: latent attention output -> per-head value space
# --------------------------------------------------------------------------
# The attention layer's output is num_heads x v_head_dim per token (page 1,
# "关键源码片段", the output_shape of the MultiHeadLatentAttentionWrapper
# excerpt), while decode attends in the latent space (page 4, "MLA Prefill vs
# Decode": W_UV is what decompresses kv_c into per-head values), so head h's
# 512-dim latent output is mapped through that head's W_UV.
def up_project_ref(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """out[r][h][v] = sum_l W_UV[h][v][l] * o_lat[r][h][l] in fp64.

    o_lat [R][H][512], w_uv [H][Vd][512] (row v of head h holds the 512 latent
    weights of value dim v) -> [R][H][Vd].
    """
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    return np.stack([np.stack([w_uv[h] @ o_lat[r, h] for h in range(o_lat.shape[1])])
                     for r in range(o_lat.shape[0])])


# --------------------------------------------------------------------------
# chunked-prefill context: paged gather with dequantisation, two-way merge
# --------------------------------------------------------------------------
# A prefill with cached context reads the context chunk by chunk: each chunk's
# latent cache rows are gathered out of the paged cache into a contiguous
# buffer and dequantised (page 4, "与非 DCP 的流程对比":
# gather_and_maybe_dequant_cache; page 2, "实现拆解" items 3 and 4, the gather
# whose requests start at seq_starts), and the chunks' partial attention
# results are merged with the LSE rule (page 4, "Chunked Prefill 与 LSE
# Merge": merge_attn_states of a prefix and a suffix result).
def gather_cache_ref(kv_cache: np.ndarray, block_table: np.ndarray, seq_starts: np.ndarray,
                     chunk_lens: np.ndarray, kv_dtype: str, kv_scale: float = 1.0) -> np.ndarray:
    """Gathered latent rows as bf16 bit patterns: [sum chunk_lens][576] uint16.

    kv_cache holds bf16 bit patterns [P][64][576] (uint16) or e4m3 codes
    (uint8).  Request b contributes its logical tokens seq_starts[b] ..
    seq_starts[b] + chunk_lens[b] - 1 (token t at row t % 64 of page
    block_table[b][t // 64]), in order, after request b - 1's.  bf16 rows are
    copied; e4m3 rows become bf16(fp32(value) * fp32(kv_scale)): the fp32
    product, rounded to nearest even.
    """
    out = []
    for b in range(len(chunk_lens)):
        t = int(seq_starts[b]) + np.arange(int(chunk_lens[b]))
        rows = kv_cache[np.asarray(block_table[b])[t // PAGE_SIZE], t % PAGE_SIZE]
        if kv_dtype == "bf16":
            out.append(np.asarray(rows).view(np.uint16))
        else:
            v = e4m3_bits_to_f64(rows).astype(np.float32) * np.float32(kv_scale)
            out.append(bf16_encode(v.astype(np.float64)))
    if not out:
        return np.zeros((0, kv_cache.shape[-1]), dtype=np.uint16)
    return np.concatenate(out, axis=0).reshape(-1, kv_cache.shape[-1])


def merge_two_ref(prefix_out, prefix_lse, suffix_out, suffix_lse):
    """merge_attn_states of a prefix and a suffix partial result: the LSE merge
    of exactly two inputs (``merge_ref`` with n = 2)."""
    return merge_ref(np.stack([prefix_out, suffix_out]), np.stack([prefix_lse, suffix_lse]))
