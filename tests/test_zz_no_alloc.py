"""mla_decode_partial_noalloc, the decode on the library's static device scratch
(for callers that cannot allocate device memory), against mla_decode_partial
with a caller workspace, through the C ABI.

Two calls in a row on the shared scratch, the second with a smaller input (so
it runs on what the first left behind): each must give the workspace entry
point's result bit for bit (same kernels, same plan) and meet the parity bars
against the fp64 oracle.  A descriptor that needs more than the scratch holds
is refused before any device work.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import compare, run_oracle, say

pytestmark = pytest.mark.gpu


def _decode(inp, noalloc: bool):
    import mla_latent_decode_absorbed_amd as mla
    desc = mla.make_desc(inp.batch, inp.q_len, inp.heads, inp.kv_cache.shape[0], inp.block_table.shape[1],
                         kv_dtype=mla.BF16 if inp.dtype == "bf16" else mla.FP8_E4M3,
                         causal=1 if inp.causal else 0)
    dev = inp.q.device
    out = torch.full((inp.batch, inp.q_len, inp.heads, 512), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((inp.batch, inp.q_len, inp.heads), float("nan"), dtype=torch.float32, device=dev)
    if noalloc:
        mla.decode_partial_noalloc(desc, inp.q, inp.kv_cache, inp.kv_scale, inp.block_table, inp.seq_lens,
                                   inp.scale, out, lse)
    else:
        mla.Decoder(desc, device=dev)(inp.q, inp.kv_cache, inp.block_table, inp.seq_lens, inp.scale,
                                      kv_scale=inp.kv_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_workspace_entry_point_on_two_calls(dtype):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 3000, size=64).tolist()
    big = workloads.make_decode_inputs(64, 1, 128, lens, dtype, seed=72, device=dev)
    small = workloads.make_decode_inputs(3, 2, 16, [37, 100, 5], dtype, seed=73, device=dev)
    for what, inp in (("first call: batch 64 x 128 heads, ragged 1..3000", big),
                      ("second, smaller call: batch 3, q_len 2, 16 heads", small)):
        say(f"noalloc {dtype}: {what}")
        o_na, l_na = _decode(inp, noalloc=True)
        o_ws, l_ws = _decode(inp, noalloc=False)
        assert torch.equal(o_na, o_ws), f"{what}: out differs from mla_decode_partial"
        assert torch.equal(l_na, l_ws), f"{what}: lse differs from mla_decode_partial"
        o_ref, l_ref = run_oracle(inp)
        compare(o_na, l_na, o_ref, l_ref, dtype=dtype, what=f"noalloc {what}")


def test_noalloc_refuses_a_descriptor_beyond_the_scratch():
    import mla_latent_decode_absorbed_amd as mla
    say("noalloc: descriptor beyond the static scratch is refused")
    dev = torch.device("cuda:0")
    inp = workloads.make_decode_inputs(2, 2, 16, [300, 200], "bf16", seed=74, device=dev)
    desc = mla.make_desc(512, 2, 128, inp.kv_cache.shape[0], 2048, num_splits=256)
    assert mla.workspace_size(desc) > mla.NOALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MlaError) as err:
        # (the size check comes first: no buffer is read, nothing is enqueued)
        mla.decode_partial_noalloc(desc, None, None, None, None, None, inp.scale, None, None)
    assert err.value.status == mla.ERR_SCRATCH_LIMIT
