"""The input generator's options that make a row's running maximum move
(logit_step, rope_ramp): checked on the logical cache rows they produce."""
import torch

import workloads

V = 512


def logical_rows(inp, b):
    """Cache rows of request b in token order, through its block table."""
    n = int(inp.seq_lens[b])
    pages = inp.block_table[b, : (n + 63) // 64].long()
    return inp.kv_cache[pages].reshape(-1, inp.kv_cache.shape[-1])[:n]


def test_logit_step_steps_the_last_key_dim():
    step = 96.0
    inp = workloads.make_decode_inputs(2, 1, 4, [1300, 700], "bf16", seed=5, logit_step=step, poison=False)
    assert torch.all(inp.q[..., -1].float() == 1.0)
    for b in range(2):
        rows = logical_rows(inp, b).float()
        t = torch.arange(rows.shape[0])
        assert torch.equal(rows[:, -1], step * torch.div(t, 512, rounding_mode="floor").float())
    # every other dim keeps the plain draw
    plain = workloads.make_decode_inputs(2, 1, 4, [1300, 700], "bf16", seed=5, poison=False)
    assert torch.equal(logical_rows(inp, 0)[:, :-1], logical_rows(plain, 0)[:, :-1])
    assert torch.equal(inp.q[..., :-1], plain.q[..., :-1])


def test_logit_step_moves_a_lazy_maximum():
    """With a step of 96, a running maximum kept in whole log2 units that moves
    only when a 32-token block's maximum exceeds it by more than 2^8 moves
    several times along 4,096 tokens in every query row (the plain draw's logits
    almost never move it after the first block)."""
    n = 4096
    inp = workloads.make_decode_inputs(1, 1, 16, [n], "bf16", seed=6, logit_step=96.0, poison=False)
    k = logical_rows(inp, 0).double()
    s = (inp.q[0, 0].double() @ k.T) * inp.scale * 1.4426950408889634   # log2 units
    for row in s:
        blocks = row.reshape(-1, 32).max(dim=1).values
        m = float(torch.ceil(blocks[0]))
        moves = 0
        for mx in blocks[1:].tolist():
            if mx > m + 8.0:
                m = float(torch.ceil(torch.tensor(mx)))
                moves += 1
        assert moves >= 3, moves


def test_rope_ramp_scales_the_rope_dims_only():
    ramp = 12.0
    n = 900
    inp = workloads.make_decode_inputs(1, 1, 4, [n], "bf16", seed=7, rope_ramp=ramp, poison=False)
    plain = workloads.make_decode_inputs(1, 1, 4, [n], "bf16", seed=7, poison=False)
    r, r0 = logical_rows(inp, 0).double(), logical_rows(plain, 0).double()
    assert torch.equal(r[:, :V], r0[:, :V])
    f = 1.0 + ramp * torch.arange(n, dtype=torch.float64) / (n - 1)
    want = r0[:, V:] * f[:, None]
    # both sides are bf16 roundings of the same fp32 value (before and after the
    # scaling): within two bf16 half-ulps of the scaled value
    assert torch.all((r[:, V:] - want).abs() <= 2 * 2.0 ** -8 * want.abs() + 1e-30)
    assert torch.equal(inp.q, plain.q)
