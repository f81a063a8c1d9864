"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the exact same bytes, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import bf16_bits_to_f64, decode_partial_ref, e4m3_bits_to_f64, merge_ref

#: max-abs-error bars: bf16 out 1e-2 and lse 1e-3; fp8 cache out 3e-2 and lse
#: 1e-3 (the fp8 LSE bar is not fixed by the method's statement; 1e-3 is the
#: bf16 bar, which the fp8 path meets: its logits are exact products of e4m3
#: codes summed in fp32, like the bf16 path's)
TOL = {"bf16": (1e-2, 1e-3), "fp8": (3e-2, 1e-3)}


def say(msg: str) -> None:
    """Name the case on stdout before any GPU work, so a fault can be attributed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def run_hip(inp, num_splits: int = 0, out_dtype=None, stream=None):
    import mla_latent_decode_absorbed_amd as mla
    if out_dtype is None:
        out_dtype = mla.F32
    desc = mla.make_desc(inp.batch, inp.q_len, inp.heads, inp.kv_cache.shape[0],
                         inp.block_table.shape[1],
                         kv_dtype=mla.BF16 if inp.dtype == "bf16" else mla.FP8_E4M3,
                         out_dtype=out_dtype, causal=1 if inp.causal else 0, num_splits=num_splits)
    dec = mla.Decoder(desc, device=inp.q.device)
    out, lse = dec(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale,
                   kv_scale=inp.kv_scale, stream=stream)
    torch.cuda.synchronize()
    return out, lse


def balanced_plan_lens():
    """128 ragged lengths (64..4000 tokens, one empty request, one of a single
    token) for which the planner's policy takes the balanced plan on an fp8
    cache with one row tile (checked by tests/test_gpu_plan.py's restatement)."""
    rng = np.random.default_rng(58)
    lens = rng.integers(64, 4000, size=128)
    lens[rng.integers(0, 128)] = 0
    lens[rng.integers(0, 128)] = 1
    return lens.tolist()


def plan_info(dec, batch: int):
    """The planner's per-request values from a decoder's workspace: int32
    [batch][4] (pieces, first piece, first global page or 0, 0)."""
    return dec.workspace[: 16 * batch].view(torch.int32).view(batch, 4).cpu().numpy()


def to_f64_q(inp, requests=None):
    q = inp.q if requests is None else inp.q[requests]
    if inp.dtype == "bf16":
        return bf16_bits_to_f64(q.view(torch.int16).cpu().numpy())
    return e4m3_bits_to_f64(q.cpu().numpy())


def cache_f64(inp, pages=None):
    kv = inp.kv_cache if pages is None else inp.kv_cache[pages]
    if inp.dtype == "bf16":
        return bf16_bits_to_f64(kv.view(torch.int16).cpu().numpy())
    return e4m3_bits_to_f64(kv.cpu().numpy())


def run_oracle(inp, requests=None):
    """Oracle on the device bytes; ``requests`` restricts to a sample (others NaN)."""
    bt = inp.block_table.cpu().numpy()
    sl = inp.seq_lens.cpu().numpy()
    if requests is None:
        q = to_f64_q(inp)
        kv = cache_f64(inp)
        return decode_partial_ref(q, kv, bt, sl, inp.scale, kv_scale=inp.kv_scale_value,
                                  causal=inp.causal)
    # copy back only the sampled requests' pages
    req = list(requests)
    pages = sorted({int(p) for b in req for p in bt[b][: (int(sl[b]) + 63) // 64]})
    remap = {p: i for i, p in enumerate(pages)}
    kv = cache_f64(inp, torch.tensor(pages, dtype=torch.long, device=inp.kv_cache.device))
    bt_s = np.full((len(req), bt.shape[1]), -1, dtype=np.int64)
    for i, b in enumerate(req):
        for j in range((int(sl[b]) + 63) // 64):
            bt_s[i, j] = remap[int(bt[b][j])]
    q = to_f64_q(inp, torch.tensor(req, dtype=torch.long, device=inp.q.device))
    return decode_partial_ref(q, kv, bt_s, sl[req], inp.scale, kv_scale=inp.kv_scale_value,
                              causal=inp.causal)


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x| (elementwise): the most a
    round-to-nearest bf16 store of a value of that magnitude can add."""
    _, e = np.frexp(np.abs(x))          # |x| in [2^(e-1), 2^e): ulp 2^(e-8)
    return np.where(x != 0, np.ldexp(1.0, e - 9), 0.0)


def compare(out, lse, o_ref, l_ref, dtype="bf16", what=""):
    """Element-by-element max-abs check of out and lse, -inf rows included.

    The bars are on the computed output; a bf16 ``out`` (an optional storage
    format) is also allowed the half ulp its own round-to-nearest store adds at
    that magnitude (up to 0.0078 at |o| in [2, 4))."""
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    tol_o, tol_l = TOL[dtype]
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    ninf_ref = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), ninf_ref), f"{what}: empty-row pattern differs"
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    diff = np.abs(o - o_ref)
    bound = tol_o + (bf16_half_ulp(np.abs(o_ref) + tol_o) if out.dtype == torch.bfloat16 else 0.0)
    err_o = float(np.max(diff)) if o.size else 0.0
    excess = float(np.max(diff - bound)) if o.size else -1.0
    fin = ~ninf_ref
    err_l = float(np.max(np.abs(l[fin] - l_ref[fin]))) if fin.any() else 0.0
    print(f"  {what}: max|dout| = {err_o:.3e} (bar {tol_o}{' + bf16 store' if out.dtype == torch.bfloat16 else ''}), "
          f"max|dlse| = {err_l:.3e} (bar {tol_l})", flush=True)
    assert excess <= 0.0, f"{what}: out error {err_o} exceeds the bar by {excess}"
    assert err_l <= tol_l, f"{what}: lse error {err_l} > {tol_l}"
    return err_o, err_l


def merge_oracle_rows(outs, lses):
    return merge_ref(np.stack(outs), np.stack(lses))
