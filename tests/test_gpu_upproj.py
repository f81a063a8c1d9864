"""GPU parity of mla_up_project (latent attention output through W_UV) against
the fp64 oracle, through the C ABI.

Bar, from the arithmetic: an fp32 input x enters as two bf16 terms with
|x - hi - lo| <= 2^-16 |x|, every bf16 product is exact in fp32, and the fp32
accumulation of at most 1024 terms adds at most 1024 * 2^-23 * sum_l |w_l x_l|.
So each element lies within delta = (2^-16 + 2^-13) * sum_l |w_l x_l| of the
exact value (a bf16 output: its code lies between the codes of exact -+ delta,
and >= 99 % equal the nearest code).  The split itself is checked too: the RMS
error must stay below 2^-14 of the RMS value, which a bf16-only input (error
~2^-9) would fail.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, bf16_encode, decode_partial_ref, up_project_ref
import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _f64(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy())
    return t.double().cpu().numpy()


def run_up(inp, out_dtype):
    import mla_latent_decode_absorbed_amd as mla
    R, H, _ = inp.o_lat.shape
    Vd = inp.w_uv.shape[1]
    out = torch.empty((R, H, Vd), dtype=out_dtype, device=DEV)
    mla.up_project(inp.o_lat, inp.w_uv, out)
    torch.cuda.synchronize()
    return out


def check_up(inp, out):
    x, w = _f64(inp.o_lat), _f64(inp.w_uv)
    exact = up_project_ref(x, w)
    absdot = up_project_ref(np.abs(x), np.abs(w))
    delta = (2.0 ** -16 + 2.0 ** -13) * absdot
    if out.dtype == torch.float32:
        got = out.double().cpu().numpy()
        err = np.abs(got - exact)
        assert (err <= delta + 1e-30).all(), float((err - delta).max())
        rms_err, rms = np.sqrt((err ** 2).mean()), np.sqrt((exact ** 2).mean())
        assert rms_err <= 2.0 ** -14 * rms, (rms_err, rms)
        return float(err.max())
    codes = out.view(torch.int16).cpu().numpy().view(np.uint16)
    g = bf16_bits_to_f64(codes)
    lo, hi = bf16_bits_to_f64(bf16_encode(exact - delta)), bf16_bits_to_f64(bf16_encode(exact + delta))
    assert ((g >= lo) & (g <= hi)).all()
    assert (codes == bf16_encode(exact)).mean() >= 0.99
    return float(np.abs(g - exact).max())


@pytest.mark.parametrize("rows,heads,vdim", [(2, 3, 128), (37, 2, 128), (5, 2, 32), (33, 2, 96),
                                             (9, 2, 160), (3, 2, 256), (4, 1, 512), (1, 5, 64)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_up_project_matches_oracle(rows, heads, vdim, in_dtype, out_dtype):
    say(f"up_project rows={rows} heads={heads} vdim={vdim} in={in_dtype} out={out_dtype}")
    inp = workloads.make_up_project_inputs(rows, heads, vdim, seed=rows * 7 + vdim, device=DEV, in_dtype=in_dtype)
    check_up(inp, run_up(inp, out_dtype))


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5"])
def test_up_project_full_size(cfg):
    c = workloads.QPREP_CONFIGS[cfg]
    say(f"up_project full size {cfg}")
    inp = workloads.make_up_project_inputs(c["rows"], c["heads"], 128, seed=9, device=DEV)
    check_up(inp, run_up(inp, torch.float32))


def test_decode_then_up_project():
    """Tiny decode on the GPU, then its latent output through W_UV; against the
    oracle's decode followed by the oracle's up-projection.  The decode's own
    error (<= 1e-2) passes through W_UV, so the bar is 1e-2 times the largest
    L1 norm of a W_UV row."""
    import mla_latent_decode_absorbed_amd as mla
    say("decode -> up_project, tiny workload")
    g, _ = workloads.make_config("c1", device=DEV)
    desc = mla.make_desc(g.batch, g.q_len, g.heads, g.kv_cache.shape[0], g.block_table.shape[1])
    o_lat, _ = mla.Decoder(desc, device=DEV)(g.q, g.kv_cache, g.block_table, g.seq_lens, g.scale)
    R = g.batch * g.q_len
    w = workloads.make_up_project_inputs(R, g.heads, 128, seed=4, device=DEV).w_uv
    out = torch.empty((R, g.heads, 128), dtype=torch.float32, device=DEV)
    mla.up_project(o_lat.view(R, g.heads, 512), w, out)
    torch.cuda.synchronize()
    o_ref, _ = decode_partial_ref(bf16_bits_to_f64(g.q.view(torch.int16).cpu().numpy()),
                                  bf16_bits_to_f64(g.kv_cache.view(torch.int16).cpu().numpy()),
                                  g.block_table.cpu().numpy(), g.seq_lens.cpu().numpy(), g.scale)
    w64 = _f64(w)
    ref = up_project_ref(o_ref.reshape(R, g.heads, 512), w64)
    bar = 1e-2 * np.abs(w64).sum(axis=-1).max()
    assert np.abs(out.double().cpu().numpy() - ref).max() <= bar


def _merge_inputs(n, R, H, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    outs = torch.randn((n, R, H, 512), generator=g)
    lses = torch.randn((n, R, H), generator=g) * 2
    if n > 1:
        lses[0, ::3] = -float("inf")                  # empty partials ...
        outs[0, ::3] = float("nan")                   # ... whose data must never be read
    lses[:, 1, 0] = -float("inf")                     # one row with every partial empty
    return outs, lses


def check_merge_up(outs, lses, w, out, lse, tokens=None):
    """The device's fused merge + up-projection against the oracle's LSE merge
    followed by its up-projection, on every token or on the sampled ``tokens``
    (all heads of each), within the bound derived in the module docstring plus
    2^-20 of the partials' spread (the fp32 weighted sum of the merge)."""
    from oracle import merge_ref
    n, R, H, _ = outs.shape
    vdim = w.shape[1]
    sel = list(range(R)) if tokens is None else list(tokens)
    T = len(sel)
    o64 = np.nan_to_num(outs[:, sel].double().cpu().numpy(), nan=0.0)
    l64 = lses[:, sel].double().cpu().numpy()
    o_m, l_m = merge_ref(o64.reshape(n, T * H, 512), l64.reshape(n, T * H))
    w64 = _f64(w)
    exact = up_project_ref(o_m.reshape(T, H, 512), w64)
    absdot = up_project_ref(np.abs(o_m).reshape(T, H, 512), np.abs(w64))
    spread = up_project_ref(np.abs(o64).sum(axis=0), np.abs(w64))
    delta = (2.0 ** -16 + 2.0 ** -13) * absdot + 2.0 ** -20 * spread
    got = out[sel].double().cpu().numpy()
    assert got.shape == (T, H, vdim)
    assert np.isfinite(got).all()
    if out.dtype == torch.float32:
        assert (np.abs(got - exact) <= delta + 1e-30).all(), float((np.abs(got - exact) - delta).max())
    else:
        lo = bf16_bits_to_f64(bf16_encode(exact - delta))
        hi = bf16_bits_to_f64(bf16_encode(exact + delta))
        assert ((got >= lo) & (got <= hi)).all()
    if lse is not None:
        gl, rl = lse[sel].double().cpu().numpy().reshape(-1), l_m
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert (np.abs(gl[fin] - rl[fin]) <= 1e-5).all()
    return got


@pytest.mark.parametrize("n,R,H,vdim", [(1, 5, 3, 128), (2, 37, 2, 128), (4, 33, 4, 96), (7, 3, 2, 160),
                                        (16, 2, 2, 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_up_project_matches_oracle(n, R, H, vdim, out_dtype):
    """mla_merge_up_project = the oracle's LSE merge followed by its up-projection."""
    import mla_latent_decode_absorbed_amd as mla
    say(f"merge_up_project n={n} R={R} H={H} vdim={vdim} {out_dtype}")
    outs, lses = _merge_inputs(n, R, H, seed=n * 100 + R)
    w = workloads.make_up_project_inputs(1, H, vdim, seed=n, device=DEV).w_uv
    out = torch.empty((R, H, vdim), dtype=out_dtype, device=DEV)
    lse = torch.empty((R, H), dtype=torch.float32, device=DEV)
    mla.merge_up_project(outs.to(DEV), lses.to(DEV), n, w, out, lse)
    torch.cuda.synchronize()
    got = check_merge_up(outs, lses, w, out, lse)
    assert (got[1, 0] == 0).all()                      # all partials empty -> 0


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_up_project_full_size_sampled(out_dtype):
    """The one-DCP-rank shape (4 shard partials of 32 tokens x 512 heads, v_head_dim
    128) against the oracle's merge + up-projection on a seeded sample of 8
    tokens with every head; the all-empty row (token 1, head 0) is in the sample."""
    import mla_latent_decode_absorbed_amd as mla
    say(f"merge_up_project full size 4 x (32 x 512), 8 sampled tokens vs oracle, {out_dtype}")
    n, R, H = 4, 32, 512
    outs, lses = _merge_inputs(n, R, H, seed=11)
    w = workloads.make_up_project_inputs(1, H, 128, seed=12, device=DEV).w_uv
    out = torch.empty((R, H, 128), dtype=out_dtype, device=DEV)
    lse = torch.empty((R, H), dtype=torch.float32, device=DEV)
    mla.merge_up_project(outs.to(DEV), lses.to(DEV), n, w, out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    tokens = sorted(set(rng.choice(R, size=7, replace=False).tolist()) | {1})
    while len(tokens) < 8:
        tokens = sorted(set(tokens) | {int(rng.integers(R))})
    got = check_merge_up(outs, lses, w, out, lse, tokens=tokens)
    assert (got[tokens.index(1), 0] == 0).all()


def test_merge_up_project_matches_unfused_full_size():
    """The one-DCP-rank shape: 4 shard partials of 32 tokens x 512 heads, fused
    against mla_merge_states followed by mla_up_project."""
    import mla_latent_decode_absorbed_amd as mla
    say("merge_up_project full size, 4 x (32 x 512)")
    n, R, H = 4, 32, 512
    outs, lses = _merge_inputs(n, R, H, seed=5)
    outs, lses = outs.to(DEV), lses.to(DEV)
    w = workloads.make_up_project_inputs(1, H, 128, seed=6, device=DEV).w_uv
    fused = torch.empty((R, H, 128), dtype=torch.float32, device=DEV)
    mla.merge_up_project(outs, lses, n, w, fused)
    merged = torch.empty((R * H, 512), dtype=torch.float32, device=DEV)
    ml = torch.empty(R * H, dtype=torch.float32, device=DEV)
    mla.merge_states(outs.reshape(n, R * H, 512).contiguous(), lses.reshape(n, R * H).contiguous(), n, R * H,
                     merged, ml)
    unfused = torch.empty((R, H, 128), dtype=torch.float32, device=DEV)
    mla.up_project(merged.view(R, H, 512), w, unfused)
    torch.cuda.synchronize()
    ref = unfused.double().cpu().numpy()
    scale = np.abs(ref).max()
    assert np.abs(fused.double().cpu().numpy() - ref).max() <= 1e-4 * scale
