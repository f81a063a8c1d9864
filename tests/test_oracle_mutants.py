"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

This shows the pins in test_oracle_pins.py are sharp enough: a dropped rope
term, the wrong V slice, log2 for ln, a missing kv_scale, a doubled scale, an
off-by-one causal limit, a wrong page slot or a wrong merge weight would not
pass unnoticed.
"""
import numpy as np
import pytest

import oracle.mla_oracle as om
import tests.test_oracle_pins as pins

pytestmark = pytest.mark.cpu


def _attend(variant):
    def f(q_rows, k_rows, v_rows, scale, kv_scale=1.0):
        R = q_rows.shape[0]
        if k_rows.shape[0] == 0:
            return np.zeros((R, v_rows.shape[-1])), np.full(R, -np.inf)
        kk = k_rows[:, :512] if variant == "drop_rope" else k_rows
        qq = q_rows[:, :512] if variant == "drop_rope" else q_rows
        sc = scale * scale if variant == "double_scale" else scale
        s = (sc * kv_scale) * (qq @ kk.T)
        mu = s.max(axis=1, keepdims=True)
        w = np.exp(s - mu)
        l = w.sum(axis=1, keepdims=True)
        lse = (mu + (np.log2(l) if variant == "log2" else np.log(l)))[:, 0]
        vv = k_rows[:, 64:576] if variant == "wrong_v" else v_rows
        o = (w / l) @ vv
        if variant != "no_kv_scale_out":
            o = kv_scale * o
        return o, lse
    return f


PIN_FUNCS = [
    lambda: pins.test_matches_torch_sdpa_fp64(37),
    pins.test_absorbed_form_equals_decompressed_mha,
    pins.test_softmax_weights_sum_to_one,
    pins.test_zero_query_gives_mean_and_log_n,
    pins.test_single_token_and_identical_keys,
    pins.test_fp8_kv_scale_enters_logits_and_output_once,
    pins.test_causal_row_equals_shorter_decode,
    pins.test_block_table_shuffle_and_nan_slack_do_not_matter,
    pins.test_any_split_point_merged_equals_whole,
    pins.test_merge_associative_permutation_invariant_identity,
    pins.test_identical_shards_add_log_d,
    lambda: pins.test_lse_merged_shards_equal_unsharded(2),
]


def _caught(monkeypatch_ctx):
    failures = 0
    for f in PIN_FUNCS:
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


@pytest.mark.parametrize("variant", ["drop_rope", "wrong_v", "log2", "no_kv_scale_out", "double_scale"])
def test_attention_mutants_are_caught(monkeypatch, variant):
    monkeypatch.setattr(om, "attend_rows", _attend(variant))
    assert _caught(monkeypatch) >= 1


def test_causal_off_by_one_is_caught(monkeypatch):
    def vis(n, q_len, causal):
        t = np.arange(q_len)
        return np.maximum(n - (q_len - t), 0) if causal else np.full(q_len, n)
    monkeypatch.setattr(om, "visible_lengths", vis)
    assert _caught(monkeypatch) >= 1


def test_wrong_page_slot_is_caught(monkeypatch):
    def gather(kv_cache, block_row, n, page_size=64):
        if n <= 0:
            return np.zeros((0, kv_cache.shape[-1]))
        j = np.arange(n)
        return kv_cache[np.asarray(block_row)[j // page_size], (page_size - 1 - j % page_size), :]
    monkeypatch.setattr(om, "gather_request_rows", gather)
    assert _caught(monkeypatch) >= 1


def test_wrong_merge_weight_is_caught(monkeypatch):
    def bad_merge(outs, lses):
        outs = np.asarray(outs, dtype=np.float64)
        lses = np.asarray(lses, dtype=np.float64)
        mu = lses.max(axis=0)
        a = np.exp(lses - mu[None])
        lse = mu + np.log(a.sum(axis=0))
        return (a[:, :, None] * outs).sum(axis=0) / outs.shape[0], lse   # averages instead of normalising
    monkeypatch.setattr(pins, "merge_ref", bad_merge)
    assert _caught(monkeypatch) >= 1
