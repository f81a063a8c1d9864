"""Pins for the fp64 oracle: what the pages and the mathematics fix, on tiny inputs.

Every check here compares the oracle with something other than itself: a
library routine (torch SDPA / logsumexp / dtype casts), the decompressed MHA
form, a closed form, a brute-force enumeration, or a value the pages print.
Each pin is chosen so that a plausible slip in the oracle (a dropped rope term,
the wrong V slice, a missing scale, log2 for ln, a wrong merge weight, an
off-by-one causal limit, a wrong page index) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    LATENT_DIM, QK_DIM, ROPE_DIM, PAGE_SIZE, absorb_query, attend_rows, bf16_bits_to_f64,
    dcp_shard_len, dcp_shard_positions, decode_partial_ref, e4m3_bits_to_f64, merge_ref,
    mha_unabsorbed_ref, visible_lengths,
)
import workloads

pytestmark = pytest.mark.cpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 1.0 / math.sqrt(192.0)


def _paged(rows_list, rng, page=PAGE_SIZE, extra=2, poison=np.nan):
    """Independent (test-side) paging of logical rows: shuffled pool, -1 past live pages."""
    pages = [(r.shape[0] + page - 1) // page for r in rows_list]
    pool = sum(pages) + extra
    perm = rng.permutation(pool)
    maxp = max(pages + [1])
    bt = -np.ones((len(rows_list), maxp), dtype=np.int64)
    cache = np.full((pool, page, rows_list[0].shape[1]), poison)
    at = 0
    for b, r in enumerate(rows_list):
        for p in range(pages[b]):
            pid = perm[at]
            at += 1
            bt[b, p] = pid
            chunk = r[p * page:(p + 1) * page]
            cache[pid, :chunk.shape[0]] = chunk
    return cache, bt


# ---------------------------------------------------------------- the pages' figures
def test_golden_page_dims():
    g = json.load(open(os.path.join(GOLDEN, "page_dims.json")))
    assert LATENT_DIM == g["kv_lora_rank"]
    assert ROPE_DIM == g["rope_dim"]
    assert QK_DIM == g["latent_width"] == g["kv_lora_rank"] + g["rope_dim"]
    assert g["mha_heads"] * g["mha_qk_dim"] == g["mha_q_values_per_token"]


# ---------------------------------------------------------------- exact decoding
def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 10).to(torch.bfloat16)
    ours = bf16_bits_to_f64(x.view(torch.int16).numpy())
    assert np.array_equal(ours, x.to(torch.float64).numpy())


# ---------------------------------------------------------------- absorbed == MHA
def test_absorbed_form_equals_decompressed_mha():
    """Decode's absorbed MQA form equals MHA over decompressed K/V (page 4, MLA Prefill vs
    Decode; page 1's W_UK_T absorption): same lse; W_UV applied to the latent output
    equals the MHA output."""
    rng = np.random.default_rng(1)
    H, n, P, R, Vd = 4, 37, 128, ROPE_DIM, 128
    w_uk = rng.standard_normal((H, P, LATENT_DIM)) / math.sqrt(LATENT_DIM)
    w_uv = rng.standard_normal((H, Vd, LATENT_DIM)) / math.sqrt(LATENT_DIM)
    q_nope = rng.standard_normal((H, P))
    q_pe = rng.standard_normal((H, R))
    kv_c = rng.standard_normal((n, LATENT_DIM))
    k_pe = rng.standard_normal((n, R))
    o_mha, lse_mha, _ = mha_unabsorbed_ref(q_nope, q_pe, kv_c, k_pe, w_uk, w_uv, SCALE)

    q_abs = absorb_query(q_nope, q_pe, w_uk)                      # [H][576]
    cache, bt = _paged([np.concatenate([kv_c, k_pe], axis=1)], rng)
    o_lat, lse = decode_partial_ref(q_abs[None, None], cache, bt, np.array([n]), SCALE)
    o_lat, lse = o_lat[0, 0], lse[0, 0]
    np.testing.assert_allclose(lse, lse_mha, rtol=1e-12, atol=0)
    o_up = np.einsum('hvl,hl->hv', w_uv, o_lat)
    np.testing.assert_allclose(o_up, o_mha, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("n", [1, 37, 100, 129])
def test_matches_torch_sdpa_fp64(n):
    rng = np.random.default_rng(2 + n)
    H = 8
    q = rng.standard_normal((1, 1, H, QK_DIM))
    rows = rng.standard_normal((n, QK_DIM))
    cache, bt = _paged([rows], rng)
    o, lse = decode_partial_ref(q, cache, bt, np.array([n]), SCALE)
    qt = torch.from_numpy(q[0, 0])[None, :, None, :]               # [1][H][1][576]
    kt = torch.from_numpy(rows)[None, None].expand(1, H, n, QK_DIM)
    vt = torch.from_numpy(rows[:, :LATENT_DIM])[None, None].expand(1, H, n, LATENT_DIM)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SCALE)
    np.testing.assert_allclose(o[0, 0], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-14)
    ref_lse = torch.logsumexp(SCALE * (qt[0, :, 0] @ kt[0, 0].T), dim=-1)
    np.testing.assert_allclose(lse[0, 0], ref_lse.numpy(), rtol=1e-12, atol=1e-14)


def test_softmax_weights_sum_to_one():
    """With every V column equal to 1 the output is sum_j w_j / l = 1 exactly (up to rounding)."""
    rng = np.random.default_rng(3)
    n, H = 77, 6
    rows = rng.standard_normal((n, QK_DIM)) * 3
    rows[:, :LATENT_DIM] = 1.0
    q = rng.standard_normal((1, 1, H, QK_DIM)) * 3
    cache, bt = _paged([rows], rng)
    o, lse = decode_partial_ref(q, cache, bt, np.array([n]), SCALE)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    # and sum_j exp(s_j - lse) = 1 with the logits recomputed from the definition
    s = SCALE * (q[0, 0] @ rows.T)
    np.testing.assert_allclose(np.exp(s - lse[0, 0][:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_and_log_n():
    rng = np.random.default_rng(4)
    n = 50
    rows = rng.standard_normal((n, QK_DIM))
    cache, bt = _paged([rows], rng)
    o, lse = decode_partial_ref(np.zeros((1, 1, 3, QK_DIM)), cache, bt, np.array([n]), SCALE)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(rows[:, :LATENT_DIM].mean(0), (3, LATENT_DIM)),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-15)


def test_single_token_and_identical_keys():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(QK_DIM)
    q = rng.standard_normal((1, 1, 4, QK_DIM))
    s0 = SCALE * (q[0, 0] @ row)
    for n in (1, 9, 64, 65):
        cache, bt = _paged([np.tile(row, (n, 1))], rng)
        o, lse = decode_partial_ref(q, cache, bt, np.array([n]), SCALE)
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(row[:LATENT_DIM], (4, LATENT_DIM)),
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], s0 + math.log(n), rtol=1e-13, atol=1e-13)


def test_empty_sequence_gives_zero_and_minus_inf():
    rng = np.random.default_rng(6)
    cache, bt = _paged([rng.standard_normal((10, QK_DIM))], rng)
    o, lse = decode_partial_ref(rng.standard_normal((1, 1, 2, QK_DIM)), cache, bt, np.array([0]), SCALE)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- merge
def _rand_partial(rng, n_tok, H=5):
    """attention of H rows over n_tok random keys: (o, lse, q, rows)"""
    q = rng.standard_normal((H, QK_DIM))
    rows = rng.standard_normal((n_tok, QK_DIM))
    o, l = attend_rows(q, rows, rows[:, :LATENT_DIM], SCALE)
    return o, l, q, rows


def test_any_split_point_merged_equals_whole():
    """Brute force over every split point of n <= 100 tokens: two partials merged = whole
    (page 4: partials over disjoint KV sets combine by LSE rescaling)."""
    rng = np.random.default_rng(7)
    for n in (2, 3, 37, 100):
        q = rng.standard_normal((4, QK_DIM))
        rows = rng.standard_normal((n, QK_DIM))
        o_all, l_all = attend_rows(q, rows, rows[:, :LATENT_DIM], SCALE)
        for k in range(0, n + 1):
            a = attend_rows(q, rows[:k], rows[:k, :LATENT_DIM], SCALE)
            b = attend_rows(q, rows[k:], rows[k:, :LATENT_DIM], SCALE)
            o, l = merge_ref(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
            np.testing.assert_allclose(o, o_all, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, l_all, rtol=1e-13, atol=1e-13)


def test_merge_associative_permutation_invariant_identity():
    rng = np.random.default_rng(8)
    parts = [_rand_partial(rng, n) for n in (5, 17, 64, 3)]
    outs = np.stack([p[0] for p in parts])
    lses = np.stack([p[1] for p in parts])
    o4, l4 = merge_ref(outs, lses)
    perm = [2, 0, 3, 1]
    op, lp = merge_ref(outs[perm], lses[perm])
    np.testing.assert_allclose(op, o4, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lp, l4, rtol=1e-14)
    oa, la = merge_ref(outs[:2], lses[:2])
    ob, lb = merge_ref(outs[2:], lses[2:])
    oab, lab = merge_ref(np.stack([oa, ob]), np.stack([la, lb]))
    np.testing.assert_allclose(oab, o4, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lab, l4, rtol=1e-14)
    o1, l1 = merge_ref(outs[:1], lses[:1])
    np.testing.assert_allclose(o1, outs[0], rtol=1e-15, atol=0)
    np.testing.assert_array_equal(l1, lses[0])


def test_merge_ignores_empty_and_all_empty():
    rng = np.random.default_rng(9)
    o, l, _, _ = _rand_partial(rng, 20)
    garbage = np.full_like(o, np.nan)
    om, lm = merge_ref(np.stack([garbage, o, garbage]),
                       np.stack([np.full_like(l, -np.inf), l, np.full_like(l, -np.inf)]))
    np.testing.assert_allclose(om, o, rtol=1e-15)
    np.testing.assert_array_equal(lm, l)
    oe, le = merge_ref(np.stack([garbage, garbage]), np.full((2, l.shape[0]), -np.inf))
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_identical_shards_add_log_d():
    rng = np.random.default_rng(10)
    o, l, _, _ = _rand_partial(rng, 33)
    for D in (2, 4, 7):
        om, lm = merge_ref(np.stack([o] * D), np.stack([l] * D))
        np.testing.assert_allclose(om, o, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lm, l + math.log(D), rtol=1e-14)


# ---------------------------------------------------------------- DCP sharding
def test_shard_length_rule_bruteforce():
    for n in range(0, 40):
        for D in (1, 2, 3, 4, 8):
            cnt = [0] * D
            for t in range(n):
                cnt[t % D] += 1
            for r in range(D):
                assert dcp_shard_len(n, D, r) == cnt[r]
                assert list(dcp_shard_positions(n, D, r)) == [t for t in range(n) if t % D == r]
                assert dcp_shard_len(n, D, r) <= -(-n // D)


@pytest.mark.parametrize("D", [2, 4])
def test_lse_merged_shards_equal_unsharded(D):
    """Each DCP rank's partial over its t mod D shard, LSE-merged, equals unsharded
    attention (page 4, DCP's role in decode: partial attention per rank, LSE-weighted merge)."""
    g, shards = workloads.make_decode_inputs(2, 1, 16, [37, 100], "bf16", seed=11, dcp=D)
    q = bf16_bits_to_f64(g.q.view(torch.int16).numpy())

    def run(inp):
        cache = bf16_bits_to_f64(inp.kv_cache.view(torch.int16).numpy())
        return decode_partial_ref(q, cache, inp.block_table.numpy(), inp.seq_lens.numpy(), g.scale)

    o_g, l_g = run(g)
    parts = [run(s) for s in shards]
    o_m, l_m = merge_ref(np.stack([p[0].reshape(-1, LATENT_DIM) for p in parts]),
                         np.stack([p[1].reshape(-1) for p in parts]))
    np.testing.assert_allclose(o_m, o_g.reshape(-1, LATENT_DIM), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_m, l_g.reshape(-1), rtol=1e-13, atol=1e-13)


def test_empty_shard_is_ignored_by_merge():
    """seq_len 1 with D = 2: shard 1 is empty (o = 0, lse = -inf); merged = shard 0 = whole."""
    g, shards = workloads.make_decode_inputs(1, 1, 4, [1], "bf16", seed=12, dcp=2)
    q = bf16_bits_to_f64(g.q.view(torch.int16).numpy())
    res = []
    for inp in [g] + shards:
        cache = bf16_bits_to_f64(inp.kv_cache.view(torch.int16).numpy())
        res.append(decode_partial_ref(q, cache, inp.block_table.numpy(), inp.seq_lens.numpy(), g.scale))
    assert np.all(np.isneginf(res[2][1])) and np.all(res[2][0] == 0)
    o_m, l_m = merge_ref(np.stack([res[1][0].reshape(-1, 512), res[2][0].reshape(-1, 512)]),
                         np.stack([res[1][1].reshape(-1), res[2][1].reshape(-1)]))
    np.testing.assert_allclose(o_m, res[0][0].reshape(-1, 512), rtol=1e-15)
    np.testing.assert_allclose(l_m, res[0][1].reshape(-1), rtol=1e-15)


# ---------------------------------------------------------------- paging
def test_block_table_shuffle_and_nan_slack_do_not_matter():
    rng = np.random.default_rng(13)
    lens = [1, 63, 64, 65, 129]
    rows = [rng.standard_normal((n, QK_DIM)) for n in lens]
    q = rng.standard_normal((len(lens), 1, 3, QK_DIM))
    # identity layout, zero slack
    maxp = max((n + 63) // 64 for n in lens)
    ident = np.zeros((len(lens) * maxp, 64, QK_DIM))
    bt_id = -np.ones((len(lens), maxp), dtype=np.int64)
    for b, r in enumerate(rows):
        for p in range((lens[b] + 63) // 64):
            bt_id[b, p] = b * maxp + p
            c = r[p * 64:(p + 1) * 64]
            ident[b * maxp + p, :c.shape[0]] = c
    o1, l1 = decode_partial_ref(q, ident, bt_id, np.array(lens), SCALE)
    cache, bt = _paged(rows, rng, poison=np.nan)          # shuffled, NaN slack + unused pages
    o2, l2 = decode_partial_ref(q, cache, bt, np.array(lens), SCALE)
    assert np.isfinite(o2).all() and np.isfinite(l2).all()
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------- fp8 scales
def test_fp8_kv_scale_enters_logits_and_output_once():
    """codes with kv_scale == their decoded values times kv_scale with kv_scale = 1."""
    inp = workloads.make_decode_inputs(2, 1, 8, [37, 100], "fp8", seed=14)
    q = e4m3_bits_to_f64(inp.q.numpy())
    codes = e4m3_bits_to_f64(inp.kv_cache.numpy())
    bt, sl = inp.block_table.numpy(), inp.seq_lens.numpy()
    o1, l1 = decode_partial_ref(q, codes, bt, sl, inp.scale, kv_scale=inp.kv_scale_value)
    o2, l2 = decode_partial_ref(q, codes * inp.kv_scale_value, bt, sl, inp.scale, kv_scale=1.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-14)
    # and the quantised problem is close to the unquantised one it came from
    assert np.isfinite(o1).all()


# ---------------------------------------------------------------- causal q_len > 1
def test_causal_row_equals_shorter_decode():
    rng = np.random.default_rng(15)
    n, H = 130, 4
    rows = rng.standard_normal((n, QK_DIM))
    cache, bt = _paged([rows], rng)
    q = rng.standard_normal((1, 2, H, QK_DIM))
    o, l = decode_partial_ref(q, cache, bt, np.array([n]), SCALE, causal=True)
    for t in range(2):
        o1, l1 = decode_partial_ref(q[:, t:t + 1], cache, bt, np.array([n - (1 - t)]), SCALE)
        np.testing.assert_array_equal(o[:, t], o1[:, 0])
        np.testing.assert_array_equal(l[:, t], l1[:, 0])
    assert list(visible_lengths(10, 3, True)) == [8, 9, 10]
    assert list(visible_lengths(10, 3, False)) == [10, 10, 10]
    on, ln_ = decode_partial_ref(q, cache, bt, np.array([n]), SCALE, causal=False)
    np.testing.assert_array_equal(on[:, 0], on[:, 0])
    assert not np.array_equal(on[:, 0], o[:, 0])
