"""GPU parity of the chunked-prefill context kernels through the C ABI:
mla_gather_cache (paged rows from seq_starts, bf16 copy or e4m3 dequantisation)
bit for bit against the oracle, and mla_merge_two_states (prefix + suffix LSE
merge) within fp32 rounding; plus a prefix and a suffix decode merged by
mla_merge_two_states against the oracle's decode over all the tokens.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, decode_partial_ref, gather_cache_ref, merge_two_ref
import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _chunks(seq_lens, rng, kind):
    """(seq_starts, chunk_lens) inside each request's tokens."""
    starts, lens = [], []
    for n in seq_lens:
        n = int(n)
        if kind == "whole":
            s, m = 0, n
        elif kind == "aligned":
            s = 64 * int(rng.integers(0, max(1, n // 64)))
            m = n - s
        elif kind == "empty_and_single":
            s, m = (n - 1, 1) if n % 2 else (0, 0)
        else:                                                   # unaligned start, random length
            s = int(rng.integers(0, max(1, n)))
            m = int(rng.integers(0, n - s + 1))
        starts.append(s)
        lens.append(m)
    return np.array(starts, dtype=np.int32), np.array(lens, dtype=np.int32)


def run_gather(inp, starts, lens):
    import mla_latent_decode_absorbed_amd as mla
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    out = torch.empty((max(total, 1), 576), dtype=torch.bfloat16, device=DEV)
    mla.gather_cache(inp.kv_cache, inp.block_table, torch.from_numpy(starts).to(DEV),
                     torch.from_numpy(cu).to(DEV), total, out, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    return out[:total].view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["whole", "aligned", "random", "empty_and_single"])
def test_gather_matches_oracle_bit_for_bit(dtype, kind):
    say(f"gather {dtype} {kind}")
    seq = [37, 100, 64, 129, 1, 300]
    inp = workloads.make_decode_inputs(len(seq), 1, 4, seq, dtype, seed=41, device=DEV)
    starts, lens = _chunks(inp.seq_lens.cpu().numpy(), np.random.default_rng(len(kind)), kind)
    got = run_gather(inp, starts, lens)
    cache = inp.kv_cache.cpu()
    cache = cache.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else cache.numpy()
    want = gather_cache_ref(cache, inp.block_table.cpu().numpy(), starts, lens, dtype, inp.kv_scale_value)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_gather_full_size_fp8():
    """Every request's first 2048 cache tokens of the fp8 workload (128 requests)."""
    say("gather fp8 full size")
    inp = workloads.make_config("c4", device=DEV, poison=False, extra_pages=0)
    sl = inp.seq_lens.cpu().numpy()
    starts = np.zeros(len(sl), dtype=np.int32)
    lens = np.minimum(sl, 2048).astype(np.int32)
    got = run_gather(inp, starts, lens)
    want = gather_cache_ref(inp.kv_cache.cpu().numpy(), inp.block_table.cpu().numpy(), starts, lens, "fp8",
                            inp.kv_scale_value)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,hd", [(1, 4), (37, 128), (300, 512), (5, 576)])
def test_merge_two_matches_oracle(in_dtype, out_dtype, rows, hd):
    import mla_latent_decode_absorbed_amd as mla
    say(f"merge_two rows={rows} hd={hd} {in_dtype} -> {out_dtype}")
    g = torch.Generator(device="cpu").manual_seed(rows * 13 + hd)
    po = torch.randn((rows, hd), generator=g).to(in_dtype)
    so = torch.randn((rows, hd), generator=g).to(in_dtype)
    pl = torch.randn(rows, generator=g) * 4
    sl = torch.randn(rows, generator=g) * 4
    pl[::5] = -float("inf")                                  # empty prefixes
    sl[::7] = -float("inf")                                  # empty suffixes (row 0: both empty)
    out = torch.empty((rows, hd), dtype=out_dtype, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    mla.merge_two_states(po.to(DEV), pl.to(DEV), so.to(DEV), sl.to(DEV), out, lse)
    torch.cuda.synchronize()
    ro, rl = merge_two_ref(po.double().numpy(), pl.double().numpy(), so.double().numpy(), sl.double().numpy())
    got = out.double().cpu().numpy()
    tol = 2e-6 + (2.0 ** -8 * np.abs(ro) if out_dtype == torch.bfloat16 else 0)
    assert (np.abs(got - ro) <= tol + 4e-6 * np.abs(ro)).all()
    gl = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert (np.abs(gl[fin] - rl[fin]) <= 1e-5).all()


def test_prefix_and_suffix_decodes_merged_equal_whole_decode():
    """Decode over each request's first 64 tokens and, with the block table
    shifted by one page, over the rest; merge_two_states of the two equals the
    oracle's decode over all the tokens (request 0 has 37 tokens: an empty
    suffix)."""
    import mla_latent_decode_absorbed_amd as mla
    say("prefix/suffix decode merge")
    g, _ = workloads.make_config("c1", device=DEV)
    n = g.seq_lens.cpu().numpy()
    rows = g.batch * g.q_len * g.heads

    def dec(bt, sl):
        desc = mla.make_desc(g.batch, g.q_len, g.heads, g.kv_cache.shape[0], bt.shape[1])
        o, l = mla.Decoder(desc, device=DEV)(g.q, g.kv_cache, bt.contiguous(), sl, g.scale)
        return o.reshape(rows, 512), l.reshape(rows)

    po, pl = dec(g.block_table, torch.from_numpy(np.minimum(n, 64).astype(np.int32)).to(DEV))
    bt_s = g.block_table[:, 1:]
    so, sl = dec(bt_s, torch.from_numpy(np.maximum(n - 64, 0).astype(np.int32)).to(DEV))
    out = torch.empty((rows, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    mla.merge_two_states(po, pl, so, sl, out, lse)
    torch.cuda.synchronize()
    o_ref, l_ref = decode_partial_ref(bf16_bits_to_f64(g.q.view(torch.int16).cpu().numpy()),
                                      bf16_bits_to_f64(g.kv_cache.view(torch.int16).cpu().numpy()),
                                      g.block_table.cpu().numpy(), n, g.scale)
    assert np.abs(out.double().cpu().numpy() - o_ref.reshape(rows, 512)).max() <= 1e-2
    assert np.abs(lse.double().cpu().numpy() - l_ref.reshape(rows)).max() <= 1e-3
