"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic split-KV unless a split count is the point).

The whole batch is decoded on the device; the fp64 oracle recomputes a seeded
sample of whole requests (every head, every query token) from the exact device
bytes, and the sampled rows are compared element by element.  The DCP rank
workload also checks the 4-shard merge at its full row count.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import merge_ref
from tests.gpu_common import compare, run_hip, run_oracle, say

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def sample(batch, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(batch, size=min(k, batch), replace=False).tolist())


def check_sampled(inp, out, lse, req, what):
    o_ref, l_ref = run_oracle(inp, requests=req)
    idx = torch.tensor(req, dtype=torch.long, device=out.device)
    compare(out[idx], lse[idx], o_ref, l_ref, dtype=inp.dtype, what=what)


def test_deepseek_v3_shape_sampled():
    """batch 64, 128 heads, seq_len 4096, bf16, automatic splits."""
    say("full-size batch64 H128 seq4096 bf16 auto splits")
    inp = workloads.make_config("c2", device=dev(), poison=True, extra_pages=5)
    out, lse = run_hip(inp)
    check_sampled(inp, out, lse, sample(inp.batch, 8, 202), "batch64/H128/4096 sampled")


def test_dcp_rank_share_and_four_shard_merge():
    """One DCP rank's share (batch 32, 512 heads, 8192 local tokens), then the
    merge of all 4 ranks' partials (16384 rows, n = 4) on the device."""
    import mla_latent_decode_absorbed_amd as mla
    req = sample(32, 8, 303)
    outs, lses, refs = [], [], []
    for r in range(4):
        say(f"full-size DCP rank {r}/4: batch32 H512 local 8192 bf16")
        sh = workloads.make_config("c3", device=dev(), poison=True, extra_pages=2, shard_only=r)
        out, lse = run_hip(sh)
        o_ref, l_ref = run_oracle(sh, requests=req)
        idx = torch.tensor(req, dtype=torch.long, device=dev())
        compare(out[idx], lse[idx], o_ref, l_ref, what=f"rank {r} sampled")
        outs.append(out.reshape(-1, 512))
        lses.append(lse.reshape(-1))
        refs.append((o_ref, l_ref))
        del sh
        torch.cuda.empty_cache()
    rows = outs[0].shape[0]
    assert rows == 32 * 512
    stk_o = torch.stack(outs).contiguous()
    stk_l = torch.stack(lses).contiguous()
    mo = torch.empty((rows, 512), dtype=torch.float32, device=dev())
    ml = torch.empty((rows,), dtype=torch.float32, device=dev())
    say("full-size 4-shard merge, 16384 rows")
    mla.merge_states(stk_o, stk_l, 4, rows, mo, ml)
    torch.cuda.synchronize()
    # (1) every row: the device merge of the device partials vs the oracle merge of the same partials
    o_m, l_m = merge_ref(stk_o.double().cpu().numpy(), stk_l.double().cpu().numpy())
    assert float(np.max(np.abs(mo.double().cpu().numpy() - o_m))) <= 1e-5
    assert float(np.max(np.abs(ml.double().cpu().numpy() - l_m))) <= 1e-5
    # (2) sampled requests end to end: merged device result vs the oracle's merged shard results
    o_ref, l_ref = merge_ref(np.stack([o.reshape(-1, 512) for o, _ in refs]),
                             np.stack([l.reshape(-1) for _, l in refs]))
    sel = torch.cat([torch.arange(b * 512, (b + 1) * 512) for b in req]).to(dev())
    compare(mo[sel], ml[sel], o_ref, l_ref, what="4-shard merge sampled")


def test_fp8_cache_sampled():
    """batch 128, 128 heads, ragged seq_lens uniform in [1024, 16384], e4m3 cache and
    query with per-tensor scales, automatic splits."""
    say("full-size fp8 batch128 H128 ragged 1024..16384 auto splits")
    inp = workloads.make_config("c4", device=dev(), poison=True, extra_pages=4)
    out, lse = run_hip(inp)
    check_sampled(inp, out, lse, sample(inp.batch, 8, 404), "fp8 batch128 sampled")


@pytest.fixture(scope="module")
def long_context():
    say("full-size long context inputs + oracle: batch4 qlen2 seq131072")
    inp = workloads.make_config("c5", device=dev(), poison=True, extra_pages=1)
    o_ref, l_ref = run_oracle(inp)
    yield inp, o_ref, l_ref
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_splits", [256, 64, 0])
def test_long_context_qlen2(long_context, num_splits):
    """batch 4, q_len 2 (causal), 128 heads, seq_len 131072: 256 and 64 chunks per
    sequence, and the automatic split, each combined on the device."""
    inp, o_ref, l_ref = long_context
    say(f"full-size long context splits={num_splits}")
    out, lse = run_hip(inp, num_splits=num_splits)
    compare(out, lse, o_ref, l_ref, what=f"long context splits={num_splits}")
