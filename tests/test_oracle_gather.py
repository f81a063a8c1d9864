"""Pins for the oracle's chunked-prefill context helpers (CPU): the paged
gather with dequantisation and the two-way LSE merge, plus planted mistakes.

The gather is pinned by an independent paging of known rows (test-side
layout, shuffled pool, NaN-free poison in unused slots), torch's casts for the
fp8 dequantisation (e4m3 -> fp32, fp32 multiply, fp32 -> bf16), and the
seq_starts offset rule.  The two-way merge is pinned by attention itself: the
merge of attention over a prefix and a suffix of the keys equals attention
over all of them (torch SDPA in fp64 as the library reference).
"""
import math

import numpy as np
import pytest
import torch

import oracle.mla_oracle as om

pytestmark = pytest.mark.cpu


def _paged(rows_list, rng, dtype_np):
    pages = [-(-r.shape[0] // 64) for r in rows_list]
    pool = sum(pages) + 3
    perm = rng.permutation(pool)
    bt = -np.ones((len(rows_list), max(pages + [1])), dtype=np.int64)
    cache = np.full((pool, 64, rows_list[0].shape[1]), 0x55, dtype=dtype_np)
    at = 0
    for b, r in enumerate(rows_list):
        for j in range(pages[b]):
            pid = perm[at]
            at += 1
            bt[b, j] = pid
            seg = r[64 * j: 64 * j + 64]
            cache[pid, :seg.shape[0]] = seg
    return cache, bt


def test_gather_bf16_copies_the_requested_token_ranges():
    rng = np.random.default_rng(31)
    lens = [100, 37, 200, 1]
    rows = [rng.integers(0, 1 << 16, (n, 576)).astype(np.uint16) for n in lens]
    cache, bt = _paged(rows, rng, np.uint16)
    starts = np.array([5, 0, 64, 0])
    chunk = np.array([70, 37, 100, 1])
    got = om.gather_cache_ref(cache, bt, starts, chunk, "bf16")
    want = np.concatenate([rows[b][starts[b]:starts[b] + chunk[b]] for b in range(4)])
    assert np.array_equal(got, want)
    empty = om.gather_cache_ref(cache, bt, starts, np.zeros(4, dtype=np.int64), "bf16")
    assert empty.shape == (0, 576)


def test_gather_fp8_dequantises_like_torch():
    rng = np.random.default_rng(32)
    lens = [130, 64]
    rows = [rng.integers(0, 256, (n, 576)).astype(np.uint8) for n in lens]
    for r in rows:
        r[(r & 0x7F) == 0x7F] = 0x12                      # no NaN codes
    cache, bt = _paged(rows, rng, np.uint8)
    starts, chunk = np.array([1, 63]), np.array([128, 1])
    scale = 0.0371
    got = om.gather_cache_ref(cache, bt, starts, chunk, "fp8", scale)
    src = np.concatenate([rows[b][starts[b]:starts[b] + chunk[b]] for b in range(2)])
    t = torch.from_numpy(src).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(scale, dtype=torch.float32)
    want = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_merge_two_of_prefix_and_suffix_equals_whole_attention():
    rng = np.random.default_rng(33)
    H, n, split, d = 3, 50, 17, 576
    q = torch.from_numpy(rng.standard_normal((H, 1, d)))
    k = torch.from_numpy(rng.standard_normal((n, d)))
    v = k[:, :512]
    scale = 1 / math.sqrt(192)

    def attend(kk, vv):
        s = scale * (q[:, 0] @ kk.T)                                     # [H][m]
        lse = torch.logsumexp(s, dim=-1)
        o = torch.nn.functional.scaled_dot_product_attention(q, kk[None].expand(H, -1, -1),
                                                             vv[None].expand(H, -1, -1), scale=scale)[:, 0]
        return o.numpy(), lse.numpy()

    po, pl = attend(k[:split], v[:split])
    so, sl = attend(k[split:], v[split:])
    wo, wl = attend(k, v)
    mo, ml = om.merge_two_ref(po, pl, so, sl)
    assert np.allclose(mo, wo, rtol=0, atol=1e-12) and np.allclose(ml, wl, rtol=0, atol=1e-12)
    eo, el = om.merge_two_ref(po, pl, np.zeros_like(so), np.full_like(sl, -np.inf))
    assert np.array_equal(eo, po) and np.allclose(el, pl, atol=1e-15)


PINS = [test_gather_bf16_copies_the_requested_token_ranges, test_gather_fp8_dequantises_like_torch,
        test_merge_two_of_prefix_and_suffix_equals_whole_attention]


def _caught():
    n = 0
    for f in PINS:
        try:
            f()
        except (AssertionError, ValueError, IndexError):
            n += 1
    return n


@pytest.mark.parametrize("variant", ["ignore_starts", "no_scale", "off_by_one_page"])
def test_gather_mutants_are_caught(monkeypatch, variant):
    good = om.gather_cache_ref

    def bad(kv_cache, block_table, seq_starts, chunk_lens, kv_dtype, kv_scale=1.0):
        if variant == "ignore_starts":
            return good(kv_cache, block_table, np.zeros_like(seq_starts), chunk_lens, kv_dtype, kv_scale)
        if variant == "off_by_one_page":
            return good(kv_cache, block_table, np.asarray(seq_starts) + 64, chunk_lens, kv_dtype, kv_scale)
        return good(kv_cache, block_table, seq_starts, chunk_lens, kv_dtype, 1.0)   # forgets the scale
    monkeypatch.setattr(om, "gather_cache_ref", bad)
    assert _caught() >= 1


def test_merge_two_weight_mutant_is_caught(monkeypatch):
    def bad(po, pl, so, sl):
        return (np.asarray(po) + np.asarray(so)) / 2, np.logaddexp(pl, sl)
    monkeypatch.setattr(om, "merge_two_ref", bad)
    assert _caught() >= 1
