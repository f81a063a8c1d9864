"""Pins for the query-preparation part of the oracle (CPU), and planted
mistakes that the pins must catch.

The prepared query is the absorbed no-rope part (W_UK_T batched matmul) joined
with the rope part, stored as bf16 or as OCP e4m3 codes under a per-tensor
query scale.  The pins compare the oracle with things other than itself:
torch's dtype casts (library routines), every finite e4m3 code, the tie and
saturation cases the formats define, a one-hot weight that fixes the weight
layout, and ``absorb_query``, which the decompressed-MHA identity pins.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
from oracle import (
    E4M3_MAX, absorb_query, bf16_bits_to_f64, bf16_encode, e4m3_bits_to_f64, e4m3_encode,
    query_prep_codes, query_prep_ref,
)

pytestmark = pytest.mark.cpu

FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_encode_round_trips_every_finite_code():
    v = e4m3_bits_to_f64(FINITE_E4M3)
    assert np.array_equal(om.e4m3_encode(v), FINITE_E4M3)


def test_e4m3_ties_go_to_even_and_off_ties_to_nearest():
    pos = FINITE_E4M3[FINITE_E4M3 < 0x80]
    vals = e4m3_bits_to_f64(pos)
    order = np.argsort(vals)
    pos, vals = pos[order], vals[order]
    for lo, hi, clo, chi in zip(vals[:-1], vals[1:], pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        even = clo if (clo & 1) == 0 else chi
        assert om.e4m3_encode(np.array([mid]))[0] == even, (lo, hi)
        d = (hi - lo) * 1e-3
        assert om.e4m3_encode(np.array([mid - d]))[0] == clo
        assert om.e4m3_encode(np.array([mid + d]))[0] == chi
        assert om.e4m3_encode(np.array([-(mid + d)]))[0] == (chi | 0x80)


def test_e4m3_saturates_at_448():
    x = np.array([448.0, 448.0 + 1e-9, 464.0, 479.9, 480.0, 1e6, np.inf, -500.0, -np.inf])
    want = np.array([0x7E] * 7 + [0xFE] * 2, dtype=np.uint8)
    assert np.array_equal(om.e4m3_encode(x), want)
    assert e4m3_bits_to_f64(np.array([0x7E], dtype=np.uint8))[0] == E4M3_MAX


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    x = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(om.e4m3_encode(x.astype(np.float64)), want)


def test_bf16_encode_matches_torch_cast_and_round_trips():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-30, 1e-3, 1.0, 1e4, 1e30)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(om.bf16_encode(x.astype(np.float64)), want)
    bits = rng.integers(0, 1 << 16, 20000).astype(np.uint16)
    bits = bits[np.isfinite(bf16_bits_to_f64(bits))]
    assert np.array_equal(om.bf16_encode(bf16_bits_to_f64(bits)), bits)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: 1 + 2^-6 wins
    got = bf16_bits_to_f64(om.bf16_encode(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])))
    assert np.array_equal(got, [1.0, 1 + 2 ** -6, -1.0])


def test_query_prep_weight_layout_one_hot():
    """w_uk_lp[h][l][p] is W_UK_T[h][p][l]: a single one at (l0, p0) copies
    q_nope[p0] into latent dim l0 of that head only."""
    R, H, P = 2, 3, 8
    rng = np.random.default_rng(13)
    qn = rng.standard_normal((R, H, P))
    qp = rng.standard_normal((R, H, 64))
    w = np.zeros((H, 512, P))
    w[1, 300, 5] = 1.0
    out = om.query_prep_ref(qn, qp, w)
    assert out.shape == (R, H, 576)
    assert np.array_equal(out[:, 1, 300], qn[:, 1, 5])
    mask = np.ones((R, H, 512), dtype=bool)
    mask[:, 1, 300] = False
    assert not out[:, :, :512][mask].any()
    assert np.array_equal(out[:, :, 512:], qp)


def test_query_prep_rows_are_absorb_query():
    R, H, P = 3, 4, 128
    rng = np.random.default_rng(14)
    qn = rng.standard_normal((R, H, P))
    qp = rng.standard_normal((R, H, 64))
    w_uk = rng.standard_normal((H, P, 512)) / np.sqrt(P)           # W_UK_T[h]: [P][512]
    out = om.query_prep_ref(qn, qp, np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1))))
    for r in range(R):
        assert np.allclose(out[r], absorb_query(qn[r], qp[r], w_uk), rtol=0, atol=1e-12)


def test_query_prep_codes_apply_the_scale_once():
    x = np.array([[[896.0, 2.0, -3.0, 1000.0]]])
    codes = query_prep_codes(x, "fp8", q_scale=2.0)
    assert np.array_equal(e4m3_bits_to_f64(codes)[0, 0], [448.0, 1.0, -1.5, 448.0])
    assert np.array_equal(query_prep_codes(x, "bf16"), om.bf16_encode(x))


# ---- planted mistakes ----------------------------------------------------
PINS = [
    test_e4m3_encode_round_trips_every_finite_code,
    test_e4m3_ties_go_to_even_and_off_ties_to_nearest,
    test_e4m3_saturates_at_448,
    test_e4m3_encode_matches_torch_cast,
    test_bf16_encode_matches_torch_cast_and_round_trips,
    test_bf16_ties_go_to_even,
    test_query_prep_weight_layout_one_hot,
    test_query_prep_rows_are_absorb_query,
]


def _caught():
    n = 0
    for f in PINS:
        try:
            with np.errstate(all="ignore"):
                f()
        except (AssertionError, ValueError, IndexError):
            n += 1
    return n


def _e4m3_variant(kind):
    good = om.e4m3_encode

    def f(x):
        x = np.asarray(x, dtype=np.float64)
        if kind == "ties_away":
            a = np.abs(x)
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
            sp = np.exp2(np.maximum(e, -6.0) - 3.0)
            q = np.floor(a / sp + 0.5) * sp
            return good(np.where(np.signbit(x), -q, q))
        if kind == "truncate":
            a = np.abs(x)
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
            sp = np.exp2(np.maximum(e, -6.0) - 3.0)
            q = np.floor(a / sp) * sp
            return good(np.where(np.signbit(x), -q, q))
        if kind == "no_saturation":
            c = good(x)
            return np.where(np.abs(x) > E4M3_MAX, np.uint8(0x7F), c).astype(np.uint8)
        if kind == "no_subnormals":
            return np.where(np.abs(x) < 2.0 ** -6, good(np.zeros_like(x)), good(x)).astype(np.uint8)
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["ties_away", "truncate", "no_saturation", "no_subnormals"])
def test_e4m3_encoder_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(om, "e4m3_encode", _e4m3_variant(kind))
    assert _caught() >= 1


def test_bf16_truncation_mutant_is_caught(monkeypatch):
    def trunc(x):
        v = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(om, "bf16_encode", trunc)
    assert _caught() >= 1


def test_transposed_weight_mutant_is_caught(monkeypatch):
    def bad(q_nope, q_pe, w_uk_lp):
        R, H, P = q_nope.shape
        w = np.asarray(w_uk_lp).reshape(H, P, 512)      # reads the latent-major array as [P][512]
        return np.stack([absorb_query(q_nope[r], q_pe[r], w) for r in range(R)])
    monkeypatch.setattr(om, "query_prep_ref", bad)
    assert _caught() >= 1
