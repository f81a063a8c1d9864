"""Pins for the oracle's output up-projection (CPU), and planted mistakes they
must catch.

up_project_ref maps each head's 512-dim latent output through W_UV.  Pinned by
the decompressed-MHA identity (the absorbed decode followed by the
up-projection equals standard attention over K/V decompressed through
W_UK/W_UV) and by a one-hot weight that fixes the weight layout.
"""
import math

import numpy as np
import pytest

import oracle.mla_oracle as om
from oracle import absorb_query, decode_partial_ref, mha_unabsorbed_ref

pytestmark = pytest.mark.cpu


def test_up_projection_of_absorbed_decode_equals_decompressed_mha():
    rng = np.random.default_rng(21)
    H, P, R_, Vd, n = 4, 128, 64, 128, 37
    q_nope = rng.standard_normal((H, P))
    q_pe = rng.standard_normal((H, R_))
    kv_c = rng.standard_normal((n, 512))
    k_pe = rng.standard_normal((n, R_))
    w_uk = rng.standard_normal((H, P, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((H, Vd, 512)) / math.sqrt(512)
    scale = 1 / math.sqrt(P + R_)
    o_mha, lse_mha, _ = mha_unabsorbed_ref(q_nope, q_pe, kv_c, k_pe, w_uk, w_uv, scale)
    q = absorb_query(q_nope, q_pe, w_uk)[None, None]                  # [1][1][H][576]
    cache = np.concatenate([kv_c, k_pe], axis=1)
    pages = -(-n // 64)
    cache_p = np.zeros((pages * 64, 576))
    cache_p[:n] = cache
    o_lat, lse = decode_partial_ref(q, cache_p.reshape(pages, 64, 576), np.arange(pages)[None], np.array([n]), scale)
    out = om.up_project_ref(o_lat.reshape(1, H, 512), w_uv)[0]
    assert np.allclose(out, o_mha, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[0, 0], lse_mha, rtol=0, atol=1e-12)


def test_up_projection_weight_layout_one_hot():
    R, H, Vd = 3, 2, 16
    rng = np.random.default_rng(22)
    o = rng.standard_normal((R, H, 512))
    w = np.zeros((H, Vd, 512))
    w[1, 5, 300] = 1.0
    out = om.up_project_ref(o, w)
    assert out.shape == (R, H, Vd)
    assert np.array_equal(out[:, 1, 5], o[:, 1, 300])
    assert np.count_nonzero(out) == R


PINS = [test_up_projection_of_absorbed_decode_equals_decompressed_mha, test_up_projection_weight_layout_one_hot]


@pytest.mark.parametrize("variant", ["transposed", "wrong_head"])
def test_up_projection_mutants_are_caught(monkeypatch, variant):
    def bad(o_lat, w_uv):
        o_lat, w_uv = np.asarray(o_lat, np.float64), np.asarray(w_uv, np.float64)
        H = o_lat.shape[1]
        if variant == "transposed":
            w = w_uv.reshape(H, 512, -1).transpose(0, 2, 1)            # reads [Vd][512] as [512][Vd]
        else:
            w = w_uv[::-1]                                             # another head's weights
        return np.stack([np.stack([w[h] @ o_lat[r, h] for h in range(H)]) for r in range(o_lat.shape[0])])
    monkeypatch.setattr(om, "up_project_ref", bad)
    caught = 0
    for f in PINS:
        try:
            f()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1
