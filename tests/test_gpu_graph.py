"""The decode path under HIP graph capture: mla_decode_partial (planning,
decode, combine) and mla_merge_states recorded into one graph and replayed
several times, with eager work and synchronisations between the replays; every
replay must reproduce the eager result bit for bit (the kernels are
deterministic, and nothing the library enqueues is a memset or a host sync)."""
import pytest
import torch

import workloads
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("cfg", ["c1", "c4"])
def test_decode_and_merge_graph_replays_match_eager(cfg):
    import mla_latent_decode_absorbed_amd as mla
    say(f"graph capture {cfg}")
    if cfg == "c1":
        g, _ = workloads.make_config("c1", device=DEV)
    else:                                                # a small fp8 batch, ragged, several splits
        g = workloads.make_decode_inputs(6, 1, 128, [1500, 64, 900, 3000, 1, 257], "fp8", seed=7, device=DEV)
    desc = mla.make_desc(g.batch, g.q_len, g.heads, g.kv_cache.shape[0], g.block_table.shape[1],
                         kv_dtype=mla.BF16 if g.dtype == "bf16" else mla.FP8_E4M3)
    dec = mla.Decoder(desc, device=DEV)
    rows = g.batch * g.q_len * g.heads
    out = torch.empty((g.batch, g.q_len, g.heads, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((g.batch, g.q_len, g.heads), dtype=torch.float32, device=DEV)
    mo = torch.empty((rows, 512), dtype=torch.float32, device=DEV)
    ml = torch.empty(rows, dtype=torch.float32, device=DEV)

    def step():
        dec(g.q, g.kv_cache, g.block_table, g.seq_lens, g.scale, kv_scale=g.kv_scale, out=out, lse=lse)
        # merge the result with itself: lse + ln 2, the same output
        mla.merge_states(torch.stack([out.view(rows, 512)] * 2), torch.stack([lse.view(rows)] * 2), 2, rows, mo, ml)

    # eager reference (the stacks above are torch copies, captured as well)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, mo, ml)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                           # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (out, lse, mo, ml):
            t.fill_(float("nan"))                        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, mo, ml), ref):
            assert torch.equal(got, want), f"replay {rep} differs"


def test_plan_once_three_layers_graph_replays_match_eager():
    """One decode step as a serving loop would capture it: mla_decode_plan once,
    then three layers' mla_decode_partial_planned on that plan (each layer its
    own query and cache); every replay reproduces the eager outputs bit for bit."""
    import mla_latent_decode_absorbed_amd as mla
    say("graph capture: plan once, three planned layers")
    base = workloads.make_decode_inputs(5, 1, 128, [700, 2100, 64, 1, 1300], "bf16", seed=71, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(72)
    layers = [(torch.randn(base.q.shape, generator=gen).to(torch.bfloat16).to(DEV),
               torch.randn(base.kv_cache.shape, generator=gen).to(torch.bfloat16).to(DEV)) for _ in range(3)]
    desc = mla.make_desc(base.batch, base.q_len, base.heads, base.kv_cache.shape[0], base.block_table.shape[1])
    dec = mla.Decoder(desc, device=DEV)
    outs = [torch.empty((base.batch, 1, base.heads, 512), dtype=torch.float32, device=DEV) for _ in layers]
    lses = [torch.empty((base.batch, 1, base.heads), dtype=torch.float32, device=DEV) for _ in layers]

    def step():
        dec.plan(base.seq_lens)
        for (q, kv), o, l in zip(layers, outs, lses):
            dec.planned(q, kv, base.block_table, base.seq_lens, base.scale, out=o, lse=l)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + lses]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs + lses:
            t.fill_(float("nan"))
        dec.workspace.fill_(0xAB)                        # the plan too is remade by every replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs + lses, ref):
            assert torch.equal(got, want), f"replay {rep} differs"
