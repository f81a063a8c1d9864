"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element; they span several 64-row M-tiles, several
pages and splits, ragged last pages (NaN-poisoned slack and unused pages),
empty sequences, q_len 2 with the causal limit, and both output dtypes.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import balanced_plan_lens, compare, plan_info, run_hip, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import mla_latent_decode_absorbed_amd  # noqa: F401  (fails loudly when not built)
    yield


def dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3])
def test_tiny_config_all_elements(num_splits):
    """Tiny workload: batch 2, 16 heads, seq_lens 37 and 100, shuffled pages, NaN slack."""
    say(f"tiny num_splits={num_splits}")
    g, _ = workloads.make_config("c1", device=dev())
    out, lse = run_hip(g, num_splits=num_splits)
    o_ref, l_ref = run_oracle(g)
    compare(out, lse, o_ref, l_ref, what=f"tiny splits={num_splits}")


def test_tiny_config_dcp2_shards_merged():
    """The same workload as two t mod 2 shards, each decoded, then merged on device."""
    import mla_latent_decode_absorbed_amd as mla
    say("tiny dcp=2 shards + merge")
    g, shards = workloads.make_config("c1", device=dev())
    outs, lses = [], []
    for sh in shards:
        o, l = run_hip(sh)
        o_ref, l_ref = run_oracle(sh)
        compare(o, l, o_ref, l_ref, what=f"shard {sh.meta['rank']}")
        outs.append(o.reshape(-1, 512))
        lses.append(l.reshape(-1))
    rows = outs[0].shape[0]
    stk_o = torch.stack(outs).contiguous()
    stk_l = torch.stack(lses).contiguous()
    mo = torch.empty((rows, 512), dtype=torch.float32, device=dev())
    ml = torch.empty((rows,), dtype=torch.float32, device=dev())
    mla.merge_states(stk_o, stk_l, len(shards), rows, mo, ml)
    torch.cuda.synchronize()
    o_ref, l_ref = run_oracle(g)
    compare(mo, ml, o_ref.reshape(rows, 512), l_ref.reshape(rows), what="merged shards vs unsharded")


@pytest.mark.parametrize("heads", [128, 20, 100])
def test_page_boundary_lengths(heads):
    """seq_lens 1, 63, 64, 65, 129 (and 0): one-token, full and ragged last pages."""
    say(f"page boundaries heads={heads}")
    inp = workloads.make_decode_inputs(6, 1, heads, [1, 63, 64, 65, 129, 0], "bf16", seed=21 + heads,
                                       device=dev())
    for ns in (0, 1, 2):
        out, lse = run_hip(inp, num_splits=ns)
        o_ref, l_ref = run_oracle(inp)
        compare(out, lse, o_ref, l_ref, what=f"boundaries H={heads} splits={ns}")
    assert torch.all(out[5] == 0) and torch.all(torch.isneginf(lse[5]))


def test_ragged_batch_many_tiles_and_splits():
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 2500, size=7).tolist()
    say(f"ragged lens={lens}")
    inp = workloads.make_decode_inputs(7, 1, 128, lens, "bf16", seed=22, device=dev())
    o_ref, l_ref = run_oracle(inp)
    for ns in (0, 1, 5, 40):
        out, lse = run_hip(inp, num_splits=ns)
        compare(out, lse, o_ref, l_ref, what=f"ragged splits={ns}")


@pytest.mark.parametrize("num_splits", [0, 3])
def test_qlen2_causal(num_splits):
    """Speculative q_len 2: query token t sees seq_len - (1 - t) tokens."""
    say(f"q_len=2 causal splits={num_splits}")
    inp = workloads.make_decode_inputs(3, 2, 128, [200, 130, 65], "bf16", seed=23, device=dev())
    assert inp.causal
    out, lse = run_hip(inp, num_splits=num_splits)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, what=f"qlen2 causal splits={num_splits}")


def test_qlen2_causal_single_token_sequence():
    """seq_len 1 with q_len 2: token 0 sees nothing (o = 0, lse = -inf), token 1 sees one."""
    say("q_len=2 causal seq_len=1")
    inp = workloads.make_decode_inputs(1, 2, 32, [1], "bf16", seed=24, device=dev())
    out, lse = run_hip(inp)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, what="qlen2 seq1")
    assert torch.isneginf(lse[0, 0]).all() and torch.all(out[0, 0] == 0)


def test_bf16_output():
    import mla_latent_decode_absorbed_amd as mla
    say("bf16 output")
    inp = workloads.make_decode_inputs(3, 1, 128, [300, 64, 1000], "bf16", seed=25, device=dev())
    o_ref, l_ref = run_oracle(inp)
    for ns in (1, 4):
        out, lse = run_hip(inp, num_splits=ns, out_dtype=mla.BF16)
        assert out.dtype == torch.bfloat16
        compare(out, lse, o_ref, l_ref, what=f"bf16 out splits={ns}")


def test_deterministic():
    say("determinism")
    inp = workloads.make_decode_inputs(4, 1, 128, [900, 1300, 40, 2048], "bf16", seed=26, device=dev())
    a = run_hip(inp)
    b = run_hip(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("n", [1, 2, 5])
def test_merge_kernel(n):
    """mla_merge_states on random partials with -inf (empty) entries, incl. all-empty rows."""
    import mla_latent_decode_absorbed_amd as mla
    from oracle import merge_ref
    say(f"merge n={n}")
    rows = 300
    g = torch.Generator().manual_seed(27 + n)
    outs = torch.randn((n, rows, 512), generator=g)
    lses = torch.randn((n, rows), generator=g) * 3
    lses[:, 7] = float("-inf")                       # all-empty row
    if n > 1:
        lses[0, 11] = float("-inf")
        outs[0, 11] = float("nan")                   # an empty partial's output is never read
    o_ref, l_ref = merge_ref(outs.double().numpy(), lses.double().numpy())
    for dt in (mla.F32, mla.BF16):
        mo = torch.empty((rows, 512), dtype=torch.float32 if dt == mla.F32 else torch.bfloat16, device=dev())
        ml = torch.empty((rows,), dtype=torch.float32, device=dev())
        mla.merge_states(outs.to(dev()), lses.to(dev()), n, rows, mo, ml, out_dtype=dt)
        torch.cuda.synchronize()
        # fp32: rounding only; bf16: one rounding to nearest (half an ulp = 2^-9 relative)
        tol = 1e-5 if dt == mla.F32 else 2.0 ** -8 * np.abs(o_ref) + 1e-6
        o = mo.double().cpu().numpy()
        l = ml.double().cpu().numpy()
        assert np.array_equal(np.isneginf(l), np.isneginf(l_ref))
        fin = ~np.isneginf(l_ref)
        assert np.all(np.abs(o - o_ref) <= tol)
        assert np.max(np.abs(l[fin] - l_ref[fin])) <= 1e-5


# ---------------------------------------------------------------------------
# OCP fp8 e4m3 cache and query (per-tensor scales: amax / 448; the query scale
# is folded into the softmax scale, the cache scale is a device float)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [0, 1, 2, 3])
def test_fp8_tiny_all_elements(num_splits):
    say(f"fp8 tiny num_splits={num_splits}")
    inp = workloads.make_decode_inputs(2, 1, 16, [37, 100], "fp8", seed=31, device=dev())
    out, lse = run_hip(inp, num_splits=num_splits)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, dtype="fp8", what=f"fp8 tiny splits={num_splits}")


@pytest.mark.parametrize("heads", [128, 20])
def test_fp8_page_boundary_lengths(heads):
    say(f"fp8 page boundaries heads={heads}")
    inp = workloads.make_decode_inputs(6, 1, heads, [1, 63, 64, 65, 129, 0], "fp8", seed=32 + heads,
                                       device=dev())
    o_ref, l_ref = run_oracle(inp)
    for ns in (0, 1, 2):
        out, lse = run_hip(inp, num_splits=ns)
        compare(out, lse, o_ref, l_ref, dtype="fp8", what=f"fp8 boundaries H={heads} splits={ns}")
    assert torch.all(out[5] == 0) and torch.all(torch.isneginf(lse[5]))


def test_fp8_ragged_many_pages_and_splits():
    rng = np.random.default_rng(33)
    lens = rng.integers(1, 3000, size=6).tolist()
    say(f"fp8 ragged lens={lens}")
    inp = workloads.make_decode_inputs(6, 1, 128, lens, "fp8", seed=33, device=dev())
    o_ref, l_ref = run_oracle(inp)
    for ns in (0, 1, 5, 30):
        out, lse = run_hip(inp, num_splits=ns)
        compare(out, lse, o_ref, l_ref, dtype="fp8", what=f"fp8 ragged splits={ns}")


@pytest.mark.parametrize("out_bf16", [False, True])
def test_fp8_balanced_plan_multi_piece_units(out_bf16):
    """Ragged fp8 batch for which the planner lays all pages end to end and
    cuts equal kv-units: workgroups run several request pieces in turn, an
    empty request gets no piece (the combine writes its zeros), and most
    requests are merged from pieces of different workgroups.  A seeded sample
    of whole requests, plus the empty and single-token ones, against the oracle."""
    import mla_latent_decode_absorbed_amd as mla
    lens = balanced_plan_lens()
    say(f"fp8 balanced plan, 128 ragged requests, {sum(lens)} tokens, bf16 out={out_bf16}")
    inp = workloads.make_decode_inputs(128, 1, 16, lens, "fp8", seed=36, device=dev())
    desc = mla.make_desc(128, 1, 16, inp.kv_cache.shape[0], inp.block_table.shape[1], kv_dtype=mla.FP8_E4M3,
                         out_dtype=mla.BF16 if out_bf16 else mla.F32)
    dec = mla.Decoder(desc, device=dev())
    out, lse = dec(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    info = plan_info(dec, 128)
    assert (info[:, 2] > 0).any(), "the balanced plan was expected"
    empty, single = lens.index(0), lens.index(1)
    assert info[empty, 0] == 0
    rng = np.random.default_rng(37)
    multi = np.nonzero(info[:, 0] > 1)[0]
    req = sorted(set(rng.choice(128, size=14, replace=False).tolist()) | {empty, single} |
                 set(rng.choice(multi, size=4, replace=False).tolist()))
    o_ref, l_ref = run_oracle(inp, requests=req)
    idx = torch.tensor(req, dtype=torch.long, device=dev())
    compare(out[idx], lse[idx], o_ref, l_ref, dtype="fp8", what=f"fp8 balanced plan bf16 out={out_bf16}")
    assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


@pytest.mark.parametrize("num_splits", [0, 3])
def test_fp8_qlen2_causal(num_splits):
    say(f"fp8 q_len=2 causal splits={num_splits}")
    inp = workloads.make_decode_inputs(3, 2, 128, [200, 130, 65], "fp8", seed=34, device=dev())
    out, lse = run_hip(inp, num_splits=num_splits)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, dtype="fp8", what=f"fp8 qlen2 causal splits={num_splits}")


def test_fp8_bf16_output_and_determinism():
    import mla_latent_decode_absorbed_amd as mla
    say("fp8 bf16 output + determinism")
    inp = workloads.make_decode_inputs(3, 1, 128, [300, 64, 1000], "fp8", seed=35, device=dev())
    o_ref, l_ref = run_oracle(inp)
    out, lse = run_hip(inp, num_splits=2, out_dtype=mla.BF16)
    assert out.dtype == torch.bfloat16
    compare(out, lse, o_ref, l_ref, dtype="fp8", what="fp8 bf16 out")
    a = run_hip(inp)
    b = run_hip(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_max_qlen16_causal_with_short_sequences(dtype):
    """q_len 16 (the largest supported) x 8 heads = one 128-row tile, causal:
    query token t sees seq_len - (15 - t) tokens, so a 5-token sequence leaves
    tokens 0..10 with nothing visible (out 0, lse -inf)."""
    say(f"q_len=16 causal {dtype}")
    inp = workloads.make_decode_inputs(3, 16, 8, [5, 16, 700], dtype, seed=41, device=dev())
    out, lse = run_hip(inp)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, dtype=dtype, what=f"qlen16 causal {dtype}")
    assert torch.isneginf(lse[0, :11]).all() and torch.all(out[0, :11] == 0)


def test_qlen4_not_causal():
    """q_len 4 with causal = 0: every query token sees every cache token."""
    say("q_len=4 not causal")
    inp = workloads.make_decode_inputs(2, 4, 32, [90, 257], "bf16", seed=42, device=dev(), causal=False)
    assert not inp.causal
    out, lse = run_hip(inp)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, what="qlen4 not causal")


@pytest.mark.parametrize("out_bf16", [False, True])
def test_forced_splits_grouped(out_bf16):
    """100 forced splits of 3 requests (300 kv-units, more than one round of
    workgroups): each workgroup runs a group of 2 consecutive splits with the
    query staged once; most splits of 2 pages cover the sequence and the rest
    are empty (lse -inf partials)."""
    import mla_latent_decode_absorbed_amd as mla
    say(f"forced splits grouped out_bf16={out_bf16}")
    inp = workloads.make_decode_inputs(3, 1, 128, [6500, 7000, 6600], "bf16", seed=45, device=dev())
    o_ref, l_ref = run_oracle(inp)
    out, lse = run_hip(inp, num_splits=100, out_dtype=mla.BF16 if out_bf16 else None)
    compare(out, lse, o_ref, l_ref, what=f"grouped splits bf16_out={out_bf16}")


def test_forced_splits_grouped_one_page_splits():
    """128 forced splits of 4 requests, q_len 2 causal (1,024 kv-units): groups
    of 4 consecutive one-page splits run as one stream, so a split ends every
    two half pages; groups hold full splits, a short last split (4 tokens)
    and empty splits after the sequence's end."""
    say("forced splits grouped, one-page splits")
    inp = workloads.make_decode_inputs(4, 2, 128, [3000, 4100, 700, 8192], "bf16", seed=46, device=dev())
    o_ref, l_ref = run_oracle(inp)
    out, lse = run_hip(inp, num_splits=128)
    compare(out, lse, o_ref, l_ref, what="grouped one-page splits")


@pytest.mark.parametrize("dtype,num_splits", [("bf16", 1), ("bf16", 0), ("bf16", 3), ("bf16", 48),
                                             ("fp8", 1), ("fp8", 0), ("fp8", 5)])
def test_reference_max_moves(dtype, num_splits):
    """Keys whose logits climb along each sequence, so that the lazy reference
    maximum of a row moves several times inside one request: bf16 (slack 2^8)
    with a logit step of 96 every 512 tokens (about 6 moves per row), fp8
    (slack 2^5) with the rope part of the keys ramped up 12-fold (about 2).
    With the plain N(0,1) inputs of the other tests it almost never moves.
    The flags in the published weights and the rescale of every wave's
    accumulators and sums all run; one piece, the auto plan, 3 splits and 48
    forced splits (grouped runs for bf16, where the maximum restarts at each
    split inside a run)."""
    say(f"reference max moves {dtype} splits={num_splits}")
    extra = dict(logit_step=96.0) if dtype == "bf16" else dict(rope_ramp=12.0)
    inp = workloads.make_decode_inputs(3, 2, 128, [3100, 3500, 4000], dtype, seed=47, device=dev(), **extra)
    o_ref, l_ref = run_oracle(inp)
    out, lse = run_hip(inp, num_splits=num_splits)
    compare(out, lse, o_ref, l_ref, dtype=dtype, what=f"max moves {dtype} splits={num_splits}")


def test_more_fixed_splits_than_pages():
    """num_splits = 8 on sequences of 1-3 pages: each request gets min(8, pages) splits."""
    say("num_splits=8, 1-3 pages")
    inp = workloads.make_decode_inputs(3, 1, 64, [40, 128, 150], "bf16", seed=43, device=dev())
    out, lse = run_hip(inp, num_splits=8)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, what="splits 8 > pages")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_three_row_tiles_partial_last(dtype):
    """q_len 3 x 100 heads = 300 rows: tiles of 128, 128 and 44 rows (the last
    tile's missing rows read a clamped query row and are never stored)."""
    say(f"300 rows {dtype}")
    inp = workloads.make_decode_inputs(2, 3, 100, [333, 64], dtype, seed=44, device=dev())
    out, lse = run_hip(inp, num_splits=2)
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, dtype=dtype, what=f"300 rows {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_out_of_pool_page_ids_are_clamped(dtype):
    """Live block-table entries outside [0, num_pages) (-1, num_pages, a large id)
    read page num_pages - 1 instead of memory outside the cache: the result
    equals the oracle's on the table with those entries replaced by
    num_pages - 1, and the requests with valid tables are unaffected."""
    import dataclasses
    say(f"out-of-pool page ids clamped, {dtype}")
    # (no NaN poison here: page num_pages - 1 may be an unused pool page)
    inp = workloads.make_decode_inputs(4, 1, 128, [200, 129, 64, 300], dtype, seed=31, device=dev(),
                                       poison=False)
    P = inp.kv_cache.shape[0]
    bt = inp.block_table.clone()
    clamped = bt.clone()
    for (b, j, bad_id) in ((0, 1, -1), (1, 0, P), (3, 4, 1 << 30)):   # live entries of requests 0, 1, 3
        bt[b, j] = bad_id
        clamped[b, j] = P - 1
    bad = dataclasses.replace(inp, block_table=bt)
    out, lse = run_hip(bad, num_splits=2)
    o_ref, l_ref = run_oracle(dataclasses.replace(inp, block_table=clamped))
    compare(out, lse, o_ref, l_ref, dtype=dtype, what=f"clamped page ids {dtype}")
    o_ok, l_ok = run_oracle(inp)
    compare(out[2:3], lse[2:3], o_ok[2:3], l_ok[2:3], dtype=dtype, what="valid-table request untouched")
