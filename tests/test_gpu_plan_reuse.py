"""The split plan made once per decode step and reused by every layer's decode
(mla_decode_plan, then mla_decode_partial_planned per layer), through the C ABI:

* on the same inputs the planned decode gives the same bytes as
  mla_decode_partial, which plans inside the call (the two planners give the
  same split list, so the decode does the same arithmetic);
* one plan serves several layers (other queries and caches, the same block
  table and seq_lens), each layer within the bars of the oracle;
* a workspace that holds no plan (never written: every work item and split
  count out of range) is skipped, not followed: out and lse stay untouched;
* past 256 requests (planner kernel instead of in-kernel planning) every row
  matches the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import balanced_plan_lens, compare, run_oracle, say

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def decoder(inp, num_splits=0, out_dtype=None):
    import mla_latent_decode_absorbed_amd as mla
    desc = mla.make_desc(inp.batch, inp.q_len, inp.heads, inp.kv_cache.shape[0], inp.block_table.shape[1],
                         kv_dtype=mla.BF16 if inp.dtype == "bf16" else mla.FP8_E4M3,
                         out_dtype=mla.F32 if out_dtype is None else out_dtype,
                         causal=1 if inp.causal else 0, num_splits=num_splits)
    return mla.Decoder(desc, device=dev())


CASES = [
    ("bf16 ragged, 3 requests x 128 heads", dict(batch=3, q_len=1, heads=128, seq_lens=[300, 64, 1000],
                                                 dtype="bf16"), 0),
    ("bf16 fixed 3 splits, 2 row tiles", dict(batch=2, q_len=2, heads=100, seq_lens=[700, 129], dtype="bf16"), 3),
    ("fp8 ragged with an empty request", dict(batch=4, q_len=1, heads=64, seq_lens=[1, 0, 2100, 640],
                                              dtype="fp8"), 0),
    ("fp8 balanced plan, 128 requests", dict(batch=128, q_len=1, heads=16, seq_lens=balanced_plan_lens(),
                                             dtype="fp8"), 0),
    ("bf16 forced 128 splits in groups of 4", dict(batch=4, q_len=2, heads=128, seq_lens=[3000, 4100, 700, 8192],
                                                   dtype="bf16"), 128),
]


@pytest.mark.parametrize("what,kw,num_splits", CASES, ids=[c[0] for c in CASES])
def test_planned_decode_equals_decode_bit_for_bit(what, kw, num_splits):
    say(f"plan reuse, same bytes: {what}")
    inp = workloads.make_decode_inputs(seed=61, device=dev(), **kw)
    a = decoder(inp, num_splits)
    out_a, lse_a = a(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, kv_scale=inp.kv_scale)
    b = decoder(inp, num_splits)
    b.workspace.fill_(0xAB)
    b.plan(inp.seq_lens)
    out_b, lse_b = b.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), f"{what}: out differs"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), f"{what}: lse differs"


@pytest.mark.parametrize("out_bf16", [False, True])
def test_one_plan_serves_three_layers(out_bf16):
    """Plan once; three layers with their own query and cache (the same block
    table and seq_lens) each match the oracle; the last layer again after the
    others, on the same plan, gives the same bytes as its first run."""
    import mla_latent_decode_absorbed_amd as mla
    say(f"plan reuse, three layers, out_bf16={out_bf16}")
    base = workloads.make_decode_inputs(3, 1, 128, [900, 1300, 40], "bf16", seed=62, device=dev())
    g = torch.Generator(device="cpu").manual_seed(63)
    layers = [dataclasses.replace(base,
                                  q=torch.randn(base.q.shape, generator=g).to(torch.bfloat16).to(dev()),
                                  kv_cache=torch.randn(base.kv_cache.shape, generator=g).to(torch.bfloat16).to(dev()))
              for _ in range(3)]
    d = decoder(base, out_dtype=mla.BF16 if out_bf16 else mla.F32)
    d.plan(base.seq_lens)
    firsts = []
    for i, inp in enumerate(layers):
        out, lse = d.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale)
        torch.cuda.synchronize()
        firsts.append((out.clone(), lse.clone()))
        o_ref, l_ref = run_oracle(inp)
        compare(out, lse, o_ref, l_ref, what=f"layer {i}")
    inp = layers[0]
    out, lse = d.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, firsts[0][0]) and torch.equal(lse, firsts[0][1])


def test_workspace_without_a_plan_is_not_followed():
    say("plan reuse, workspace never planned")
    inp = workloads.make_decode_inputs(2, 1, 16, [37, 100], "bf16", seed=64, device=dev())
    d = decoder(inp)
    d.workspace.fill_(0xAB)           # every work item and split count negative
    out = torch.full((inp.batch, 1, inp.heads, 512), 7.0, dtype=torch.float32, device=dev())
    lse = torch.full((inp.batch, 1, inp.heads), 5.0, dtype=torch.float32, device=dev())
    d.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 5.0).all())
    # planning into the same workspace afterwards makes it usable
    d.plan(inp.seq_lens)
    out, lse = d.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, what="after planning")
    assert np.isfinite(lse.cpu().numpy()).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_batch_past_the_fused_planner_matches_oracle(dtype):
    """300 requests (more than the decode kernel plans for itself): the planner
    kernel writes the split list, the decode follows it.  Every row against the
    oracle; ragged lengths 0..400 with empty requests; the stored-plan call
    gives the same bytes."""
    say(f"batch 300 through the planner kernel, {dtype}")
    rng = np.random.default_rng(66)
    lens = rng.integers(0, 401, size=300)
    lens[rng.choice(300, size=9, replace=False)] = 0
    inp = workloads.make_decode_inputs(300, 1, 16, lens.tolist(), dtype, seed=67, device=dev())
    d = decoder(inp)
    out, lse = d(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    o_ref, l_ref = run_oracle(inp)
    compare(out, lse, o_ref, l_ref, dtype=dtype, what=f"batch 300 {dtype}")
    d.plan(inp.seq_lens)
    out2, lse2 = d.planned(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
