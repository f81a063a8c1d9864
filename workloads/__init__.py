"""Seeded synthetic inputs for absorbed-MQA MLA decode over a paged latent cache.

This module is shared by the parity tests, the benchmark and the oracle checks.
It holds none of the method's arithmetic: it draws N(0, 1) values, rounds them
to bf16 or quantises them to OCP e4m3 with a per-tensor scale, lays token rows
out in 64-token pages behind a shuffled block table, and splits a sequence into
DCP shards by t -> t mod D.  PyTorch is used for the draws and the dtype casts.

Recipe (one per call, seeded):
  1. q ~ N(0, 1) as [B][q_len][H][576] (fp32 draw);
  2. per request b, logical cache rows ~ N(0, 1) as [seq_len_b][576];
  3. bf16: round to nearest even; fp8: scale = amax / 448 over the tensor
     (q and cache separately), codes = e4m3fn(x / scale) (RNE, saturating);
  4. block table: a random permutation of the page pool; request b takes the
     next ceil(n_b / 64) page ids; the rest of its row is -1;
  5. slack rows of each last page and unused pool pages hold NaN (parity
     runs, ``poison=True``) or zero (timing runs).
The workloads named by ``CONFIGS`` follow the page's shapes: DeepSeek-style
128 heads of 576 = 512 latent + 64 rope, softmax scale 1/sqrt(192).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

QK_DIM = 576
V_DIM = 512
PAGE = 64
E4M3_MAX = 448.0
#: the softmax scale of the workloads: 1/sqrt(qk_nope + qk_rope) = 1/sqrt(128 + 64)
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

CONFIGS = {
    # tiny: the oracle's own case, also sharded D = 2 by t mod 2
    "c1": dict(batch=2, q_len=1, heads=16, seq_lens=[37, 100], dtype="bf16", dcp=2),
    # DeepSeek-V3 shape on one unsharded cache
    "c2": dict(batch=64, q_len=1, heads=128, seq_lens=4096, dtype="bf16", dcp=1),
    # one DCP rank's share: 512 = 128 x 4 heads, 8192 local tokens of 32768
    "c3": dict(batch=32, q_len=1, heads=512, seq_lens=32768, dtype="bf16", dcp=4),
    # fp8 cache, ragged lengths uniform in [1024, 16384]
    "c4": dict(batch=128, q_len=1, heads=128, seq_lens=(1024, 16384), dtype="fp8", dcp=1),
    # long context, low concurrency, speculative q_len 2
    "c5": dict(batch=4, q_len=2, heads=128, seq_lens=131072, dtype="bf16", dcp=1),
}


@dataclass
class DecodeInputs:
    """One shard's decode inputs, as laid out in device memory."""
    q: torch.Tensor              # [B][q_len][H][576] bfloat16, or uint8 e4m3 codes
    kv_cache: torch.Tensor       # [P][64][576] bfloat16, or uint8 e4m3 codes
    block_table: torch.Tensor    # int32 [B][max_pages], -1 past the live pages
    seq_lens: torch.Tensor       # int32 [B]
    scale: float                 # softmax scale (query scale folded in for fp8)
    dtype: str                   # "bf16" | "fp8"
    causal: bool
    kv_scale_value: float = 1.0  # per-tensor cache scale (fp8), 1 for bf16
    q_scale_value: float = 1.0   # per-tensor query scale (fp8), 1 for bf16
    kv_scale: torch.Tensor | None = None   # float32 [1] on the device (fp8)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def q_len(self) -> int:
        return self.q.shape[1]

    @property
    def heads(self) -> int:
        return self.q.shape[2]


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round to bfloat16, nearest even (torch's cast)."""
    return x.to(torch.bfloat16)


def quantize_e4m3(xs, amax: float | None = None):
    """Per-tensor OCP e4m3fn quantisation: scale = amax / 448, codes = e4m3(x / scale).

    ``xs`` is a tensor or a list of tensors sharing one scale.  Returns
    (codes as uint8 tensors of the same structure, scale as a Python float).
    """
    many = isinstance(xs, (list, tuple))
    lst = list(xs) if many else [xs]
    if amax is None:
        amax = max((float(x.abs().max()) for x in lst if x.numel() > 0), default=1.0)
    scale = float(torch.tensor(amax / E4M3_MAX, dtype=torch.float32))
    if scale == 0.0:
        scale = 1.0
    codes = [(x.float() / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
             for x in lst]
    return (codes if many else codes[0]), scale


def page_layout(seq_lens, gen_cpu: torch.Generator, extra_pages: int = 0,
                max_pages: int | None = None):
    """Shuffled page ids for each request.  Returns (block_table int32 [B][maxp], pool size)."""
    pages = [(int(n) + PAGE - 1) // PAGE for n in seq_lens]
    pool = sum(pages) + int(extra_pages)
    maxp = max(pages + [1]) if max_pages is None else int(max_pages)
    perm = torch.randperm(max(pool, 1), generator=gen_cpu).to(torch.int32)
    bt = torch.full((len(pages), maxp), -1, dtype=torch.int32)
    at = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[at:at + p]
        at += p
    return bt, max(pool, 1)


def scatter_pages(rows, block_table: torch.Tensor, pool: int, dtype, poison: bool, device):
    """Write each request's logical rows into its pages of a fresh [pool][64][576] cache."""
    if dtype == torch.uint8:
        fill = 0x7F if poison else 0          # 0x7F is an e4m3fn NaN code
    else:
        fill = float("nan") if poison else 0.0
    cache = torch.full((pool, PAGE, QK_DIM), fill, dtype=dtype, device=device)
    bt_dev = block_table.to(device=device, dtype=torch.long)
    for b, r in enumerate(rows):
        n = r.shape[0]
        if n == 0:
            continue
        p = (n + PAGE - 1) // PAGE
        padded = torch.full((p * PAGE, QK_DIM), fill, dtype=cache.dtype, device=device)
        padded[:n] = r
        cache[bt_dev[b, :p]] = padded.view(p, PAGE, QK_DIM)
    return cache


def _seq_lens_for(cfg: dict, gen_cpu: torch.Generator):
    B = cfg["batch"]
    sl = cfg["seq_lens"]
    if isinstance(sl, int):
        return [sl] * B
    if isinstance(sl, tuple):
        lo, hi = sl
        return torch.randint(lo, hi + 1, (B,), generator=gen_cpu).tolist()
    assert len(sl) == B
    return list(sl)


def make_decode_inputs(batch: int, q_len: int, heads: int, seq_lens, dtype: str = "bf16",
                       seed: int = 0, device="cpu", poison: bool = True, extra_pages: int = 3,
                       scale: float = DEFAULT_SCALE, causal: bool | None = None,
                       dcp: int = 1, max_pages: int | None = None, rope_ramp: float = 0.0,
                       logit_step: float = 0.0):
    """Inputs for one cache, or for D DCP shards of one logical cache.

    Returns a DecodeInputs when dcp == 1, else (global DecodeInputs, [shard DecodeInputs]).
    Shard r holds the global tokens t with t mod D == r, in order, in its own
    shuffled pool; all shards and the global cache see the same query.

    rope_ramp > 0 multiplies the rope part (the last 64 dims) of token t of a
    request of n tokens by 1 + rope_ramp * t / (n - 1) before storage, so that
    the logits' spread, and with it the running row maximum, grows along the
    sequence (the values, the first 512 dims, keep their distribution).

    logit_step > 0 sets the last query dim to 1 and the last key dim of token t
    to logit_step * floor(t / 512): every 512 tokens every row's logits rise by
    scale * logit_step, so the running maximum of every row moves several times
    along a long sequence while the softmax stays as spread as without it.
    """
    assert dtype in ("bf16", "fp8")
    seq_lens = [int(n) for n in seq_lens]
    assert len(seq_lens) == batch
    if causal is None:
        causal = q_len > 1
    gen_cpu = make_generator(seed, "cpu")
    gen_dev = make_generator(seed + 1_000_003, device)
    q32 = torch.randn((batch, q_len, heads, QK_DIM), generator=gen_dev, device=device)
    rows32 = [torch.randn((n, QK_DIM), generator=gen_dev, device=device) for n in seq_lens]
    if logit_step > 0:
        q32[..., -1] = 1.0
        for r in rows32:
            r[:, -1] = logit_step * torch.div(torch.arange(r.shape[0], device=device), 512,
                                              rounding_mode="floor").to(torch.float32)
    if rope_ramp > 0:
        for r in rows32:
            n = r.shape[0]
            if n > 1:
                f = 1.0 + rope_ramp * torch.arange(n, device=device, dtype=torch.float32) / (n - 1)
                r[:, V_DIM:] *= f[:, None]

    if dtype == "bf16":
        q = to_bf16(q32)
        rows = [to_bf16(r) for r in rows32]
        q_scale = kv_scale = 1.0
        el = torch.bfloat16
        eff_scale = scale
    else:
        q, q_scale = quantize_e4m3(q32)
        rows, kv_scale = quantize_e4m3(rows32)
        el = torch.uint8
        eff_scale = float(torch.tensor(scale * q_scale, dtype=torch.float32))
    del q32, rows32

    def one(rows_list, seed_off):
        g = make_generator(seed * 7919 + seed_off, "cpu")
        lens = [r.shape[0] for r in rows_list]
        bt, pool = page_layout(lens, g, extra_pages=extra_pages, max_pages=max_pages)
        cache = scatter_pages(rows_list, bt, pool, el, poison, device)
        ks = None
        if dtype == "fp8":
            ks = torch.tensor([kv_scale], dtype=torch.float32, device=device)
        return DecodeInputs(q=q, kv_cache=cache, block_table=bt.to(device),
                            seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                            scale=eff_scale, dtype=dtype, causal=causal,
                            kv_scale_value=kv_scale, q_scale_value=q_scale, kv_scale=ks)

    if dcp == 1:
        return one(rows, 1)
    glob = one(rows, 1)
    shards = [one([r[s::dcp] for r in rows], 2 + s) for s in range(dcp)]
    for s, sh in enumerate(shards):
        sh.meta.update(dcp=dcp, rank=s)
    return glob, shards


def make_config(name: str, seed: int | None = None, device="cpu", poison: bool = True,
                extra_pages: int = 3, shard_only: int | None = None):
    """The named workload.  Seed defaults to the config number.

    c1 and c3 are DCP-sharded: returns (global, shards).  For c3 the global
    cache is large; ``shard_only=r`` builds only shard r's inputs (the shards
    then get independent draws of their own tokens).
    """
    cfg = CONFIGS[name]
    if seed is None:
        seed = int(name[1:])
    gen_cpu = make_generator(seed, "cpu")
    lens = _seq_lens_for(cfg, gen_cpu)
    D = cfg["dcp"]
    if D > 1 and shard_only is not None:
        r = int(shard_only)
        local = [max(0, (n - r + D - 1) // D) for n in lens]
        inp = make_decode_inputs(cfg["batch"], cfg["q_len"], cfg["heads"], local, cfg["dtype"],
                                 seed=seed * 31 + r, device=device, poison=poison,
                                 extra_pages=extra_pages)
        inp.meta.update(dcp=D, rank=r, global_seq_lens=lens)
        return inp
    return make_decode_inputs(cfg["batch"], cfg["q_len"], cfg["heads"], lens, cfg["dtype"],
                              seed=seed, device=device, poison=poison, extra_pages=extra_pages,
                              dcp=D)


# ---------------------------------------------------------------------------
# query preparation inputs
# ---------------------------------------------------------------------------
@dataclass
class QueryPrepInputs:
    """Inputs of the query preparation (absorption + rope concat + storage)."""
    q_nope: torch.Tensor     # [R][H][P] bfloat16
    q_pe: torch.Tensor       # [R][H][64] bfloat16
    w_uk: torch.Tensor       # [H][512][P] bfloat16, w_uk[h][l][p] = W_UK_T[h][p][l]
    q_scale: torch.Tensor | None   # device float[1] for e4m3 output, else None
    q_scale_value: float


#: query-preparation shapes: the query rows and heads of the decode workloads
#: (rows = batch x q_len), DeepSeek's no-rope width P = 128
QPREP_CONFIGS = {
    "c1": dict(rows=2, heads=16),
    "c2": dict(rows=64, heads=128),
    "c3": dict(rows=32, heads=512),
    "c4": dict(rows=128, heads=128),
    "c5": dict(rows=8, heads=128),
}


def make_query_prep_inputs(rows: int, heads: int, nope_dim: int = 128, seed: int = 0, device="cpu",
                           fp8: bool = False, q_scale: float = 1.0 / 64.0) -> QueryPrepInputs:
    """Seeded query-preparation inputs: q_nope and q_pe ~ N(0, 1), W_UK_T ~ N(0, 1/P)
    (so that the absorbed values are about N(0, 1), like the decode workloads'
    query), all rounded to bf16; the weights are laid out latent-major.  The
    fp8 query scale is a fixed input (a calibrated per-tensor scale in a
    model); the default 1/64 represents magnitudes up to 7."""
    gen = make_generator(seed, device)
    qn = torch.randn((rows, heads, nope_dim), generator=gen, device=device)
    qp = torch.randn((rows, heads, 64), generator=gen, device=device)
    w_t = torch.randn((heads, nope_dim, V_DIM), generator=gen, device=device) / math.sqrt(nope_dim)
    w = w_t.transpose(1, 2).contiguous()
    qs = torch.tensor([q_scale], dtype=torch.float32, device=device) if fp8 else None
    return QueryPrepInputs(to_bf16(qn), to_bf16(qp), to_bf16(w), qs, float(q_scale))


# ---------------------------------------------------------------------------
# output up-projection inputs
# ---------------------------------------------------------------------------
@dataclass
class UpProjectInputs:
    o_lat: torch.Tensor      # [R][H][512] float32 or bfloat16 (latent attention output)
    w_uv: torch.Tensor       # [H][Vd][512] bfloat16


def make_up_project_inputs(rows: int, heads: int, vdim: int = 128, seed: int = 0, device="cpu",
                           in_dtype: str = "f32") -> UpProjectInputs:
    """Seeded up-projection inputs: the latent output ~ N(0, 1) in fp32 (or
    rounded to bf16), W_UV ~ N(0, 1/512) rounded to bf16, laid out [H][Vd][512]."""
    gen = make_generator(seed, device)
    o = torch.randn((rows, heads, V_DIM), generator=gen, device=device)
    w = torch.randn((heads, vdim, V_DIM), generator=gen, device=device) / math.sqrt(V_DIM)
    if in_dtype == "bf16":
        o = to_bf16(o)
    return UpProjectInputs(o.contiguous(), to_bf16(w).contiguous())
