"""GPU parity of mla_query_prep (absorption through W_UK_T, rope concat, bf16 or
e4m3 storage) against the fp64 oracle, through the C ABI.

The stored value is an integer code decided by rounding a floating-point sum,
and the kernel's fp32 MFMA sum differs from the exact sum by at most
gamma = 2 P 2^-24 sum_p |q_p w_p| (fp32 accumulation of exact bf16 products).
Where the exact value lies within gamma of a rounding boundary both neighbouring
codes are correct, so each element must hold a code between the codes of
(exact - gamma) and (exact + gamma); elsewhere that range is one code and the
check is exact.  At least 99.9 % of the latent codes must equal the oracle's
code of the exact value, and the rope part (no arithmetic but the fp8
division) must match bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import (
    bf16_bits_to_f64, bf16_encode, decode_partial_ref, e4m3_bits_to_f64, e4m3_encode,
    query_prep_codes, query_prep_ref,
)
import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _f64(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy())


def run_prep(inp):
    import mla_latent_decode_absorbed_amd as mla
    R, H, _ = inp.q_nope.shape
    fp8 = inp.q_scale is not None
    out = torch.empty((R, H, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
    mla.query_prep(inp.q_nope, inp.q_pe, inp.w_uk, out, q_scale=inp.q_scale)
    torch.cuda.synchronize()
    return out


def check_prep(inp, out):
    fp8 = inp.q_scale is not None
    qn, qp, w = _f64(inp.q_nope), _f64(inp.q_pe), _f64(inp.w_uk)
    exact = query_prep_ref(qn, qp, w)                                   # [R][H][576]
    P = qn.shape[-1]
    absdot = np.einsum('rhp,hlp->rhl', np.abs(qn), np.abs(w))
    gamma = np.concatenate([2 * P * 2.0 ** -24 * absdot, np.zeros(qp.shape)], axis=-1)
    if fp8:
        qs = inp.q_scale_value
        got_codes = out.cpu().numpy()
        want = query_prep_codes(exact, "fp8", qs)
        lo_v, hi_v = (exact - gamma) / qs, (exact + gamma) / qs
        pad = 2.0 ** -23 * np.abs(exact / qs)                           # the fp32 division's rounding
        lo, hi = e4m3_encode(lo_v - pad), e4m3_encode(hi_v + pad)
        dec = e4m3_bits_to_f64
    else:
        got_codes = out.view(torch.int16).cpu().numpy().view(np.uint16)
        want = query_prep_codes(exact, "bf16")
        lo, hi = bf16_encode(exact - gamma), bf16_encode(exact + gamma)
        dec = bf16_bits_to_f64
    g, lo_d, hi_d = dec(got_codes), dec(lo), dec(hi)
    bad = ~((g >= lo_d) & (g <= hi_d))
    assert not bad.any(), (f"{int(bad.sum())} codes outside the valid range; first at "
                           f"{np.argwhere(bad)[0]}: got {g[bad][0]}, range [{lo_d[bad][0]}, {hi_d[bad][0]}]")
    same = (got_codes[..., :512] == want[..., :512]).mean()
    assert same >= 0.999, same
    assert np.array_equal(got_codes[..., 512:], want[..., 512:])
    return same


@pytest.mark.parametrize("rows,heads,P", [(2, 16, 128), (37, 5, 128), (33, 3, 64), (5, 2, 192),
                                          (31, 2, 256), (64, 1, 16), (1, 7, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_query_prep_matches_oracle(rows, heads, P, dtype):
    say(f"query_prep rows={rows} heads={heads} P={P} {dtype}")
    inp = workloads.make_query_prep_inputs(rows, heads, P, seed=rows * 31 + heads, device=DEV,
                                           fp8=dtype == "fp8", q_scale=0.0173)
    check_prep(inp, run_prep(inp))


@pytest.mark.parametrize("q_scale", [64.0, 1.0 / 256.0])
def test_query_prep_fp8_subnormal_and_saturating_scales(q_scale):
    """q_scale 64 puts most values in e4m3's subnormal range; 1/256 saturates
    every magnitude above 1.75."""
    say(f"query_prep fp8 q_scale={q_scale}")
    inp = workloads.make_query_prep_inputs(40, 8, 128, seed=7, device=DEV, fp8=True, q_scale=q_scale)
    out = run_prep(inp)
    check_prep(inp, out)
    codes = out.cpu().numpy()
    if q_scale > 1:
        assert ((codes & 0x78) == 0).mean() > 0.5          # exponent field 0: subnormal (or zero)
    else:
        assert ((codes & 0x7F) == 0x7E).mean() > 0.05      # +-448


@pytest.mark.parametrize("cfg,dtype", [("c2", "bf16"), ("c3", "bf16"), ("c4", "fp8"), ("c5", "bf16")])
def test_query_prep_full_size(cfg, dtype):
    """The query rows and heads of each decode workload, at full size."""
    c = workloads.QPREP_CONFIGS[cfg]
    say(f"query_prep full size {cfg} {dtype}")
    inp = workloads.make_query_prep_inputs(c["rows"], c["heads"], 128, seed=5, device=DEV,
                                           fp8=dtype == "fp8")
    check_prep(inp, run_prep(inp))


def test_query_prep_rejects_bad_shapes():
    import mla_latent_decode_absorbed_amd as mla
    inp = workloads.make_query_prep_inputs(4, 2, 128, seed=1, device=DEV)
    out = torch.empty((4, 2, 576), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        mla.query_prep(inp.q_nope, inp.q_pe, inp.w_uk[:, :, :64].contiguous(), out)
    with pytest.raises(ValueError):
        mla.query_prep(inp.q_nope, inp.q_pe, inp.w_uk, out[:3])
    with pytest.raises(mla.MlaError):      # P = 136 is not a multiple of 16
        qn = torch.zeros((4, 2, 136), dtype=torch.bfloat16, device=DEV)
        mla.query_prep(qn, inp.q_pe, torch.zeros((2, 512, 136), dtype=torch.bfloat16, device=DEV), out)


def test_prepared_query_feeds_the_decode():
    """Prepared query (bf16) -> decode on the GPU, against the oracle's decode of
    the oracle's prepared query: the two steps together stay within the decode's
    bars."""
    import mla_latent_decode_absorbed_amd as mla
    say("query_prep -> decode, tiny workload")
    g, _ = workloads.make_config("c1", device=DEV)
    R, H = g.batch * g.q_len, g.heads
    inp = workloads.make_query_prep_inputs(R, H, 128, seed=3, device=DEV)
    q = run_prep(inp).view(g.batch, g.q_len, H, 576)
    desc = mla.make_desc(g.batch, g.q_len, H, g.kv_cache.shape[0], g.block_table.shape[1])
    out, lse = mla.Decoder(desc, device=DEV)(q, g.kv_cache, g.block_table, g.seq_lens, g.scale)
    torch.cuda.synchronize()
    q_ref = bf16_bits_to_f64(query_prep_codes(query_prep_ref(_f64(inp.q_nope), _f64(inp.q_pe), _f64(inp.w_uk)),
                                              "bf16")).reshape(g.batch, g.q_len, H, 576)
    o_ref, l_ref = decode_partial_ref(q_ref, _f64(g.kv_cache), g.block_table.cpu().numpy(),
                                      g.seq_lens.cpu().numpy(), g.scale)
    assert np.abs(out.double().cpu().numpy() - o_ref).max() <= 1e-2
    assert np.abs(lse.double().cpu().numpy() - l_ref).max() <= 1e-3
