"""The device planner's split list, checked integer for integer.

The planner (one workgroup, no host sync) reads seq_lens on the device and
writes, into the workspace, per request its split count and first kv-unit, and
the list of work items the decode kernel runs.  Which split list it picks only
moves time around, so an error in it would show up as lost speed, not as a
parity failure; this test reads the list back and compares it with the policy
restated below in plain Python:

* a request of n cache tokens has P = ceil(n / 64) pages;
* num_splits = k > 0: max(1, min(k, P)) splits of ceil(P / S) pages;
* automatic: the smallest chunk c (pages) with c >= max(2, ceil(sum P / U))
  such that sum_b max(1, ceil(P_b / c)) <= U, where U = max(1, target // m_tiles)
  and target = min(compute units, 256); if no chunk up to the longest request
  fits, every request gets one split;
* split s of request b covers pages [min(P, s c), min(P, (s + 1) c));
* kv-units are numbered request by request, split by split (K in all); with
  C = ceil(K / 8), work slot u holds kv-unit k = C (u % 8) + (u // 8) // m_tiles
  and row tile (u // 8) % m_tiles, or is empty when (u // 8) // m_tiles >= C or
  k >= K (the XCD-contiguous order: slot u runs on XCD u % 8).

The workspace layout read here is the library's internal one: int32 [B][2]
(splits, first kv-unit) at offset 0, then 32-byte work items (b, mt, split,
page_begin, page_end, nsplit, 0, 0) at the next 256-byte boundary.
"""
import numpy as np
import pytest
import torch

from tests.gpu_common import say

pytestmark = pytest.mark.gpu

PAGE = 64
MIN_CHUNK = 2
TARGET_CAP = 256
M_TILE = 128


def pages_of(seq_lens, max_pages):
    n = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, max_pages * PAGE)
    return (n + PAGE - 1) // PAGE


def expected_plan(seq_lens, max_pages, m_tiles, num_splits, target):
    pg = pages_of(seq_lens, max_pages)
    B = len(pg)
    if num_splits > 0:
        S = np.maximum(1, np.minimum(num_splits, pg))
        cb = (pg + S - 1) // S
    else:
        cap = max(1, target // m_tiles)
        start = max(MIN_CHUNK, -(-int(pg.sum()) // cap))
        longest = max(1, int(pg.max()))
        chunk = None
        for c in range(start, longest + 1):
            if int(np.maximum(1, (pg + c - 1) // c).sum()) <= cap:
                chunk = c
                break
        if chunk is None:
            chunk = max(start, longest)
        S = np.maximum(1, (pg + chunk - 1) // chunk)
        cb = np.full(B, chunk, dtype=np.int64)
    first = np.concatenate([[0], np.cumsum(S)[:-1]])
    units = []
    for b in range(B):
        for s in range(int(S[b])):
            units.append((b, s, min(pg[b], s * cb[b]), min(pg[b], (s + 1) * cb[b]), int(S[b])))
    return S, first, units


def units_max(B, m_tiles, max_pages, num_splits):
    if num_splits > 0:
        k = B * max(1, min(num_splits, max_pages))
    else:
        k = TARGET_CAP // m_tiles + B
    return ((k + 7) // 8) * 8 * m_tiles


def run_plan(seq_lens, heads, q_len, max_pages, num_splits):
    import mla_latent_decode_absorbed_amd as mla
    dev = torch.device("cuda:0")
    B = len(seq_lens)
    pool = 4
    g = torch.Generator().manual_seed(1234 + B)
    q = (torch.randn((B, q_len, heads, 576), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kv = (torch.randn((pool, PAGE, 576), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    bt = torch.randint(0, pool, (B, max_pages), generator=g, dtype=torch.int32).to(dev)
    sl = torch.tensor(seq_lens, dtype=torch.int32).to(dev)
    desc = mla.make_desc(B, q_len, heads, pool, max_pages, num_splits=num_splits)
    dec = mla.Decoder(desc, device=dev)
    dec.workspace.fill_(0xAB)
    out, lse = dec(q, kv, bt, sl, 0.07)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ws = dec.workspace.cpu().numpy()
    req = ws[:8 * B].view(np.int32).reshape(B, 2)
    woff = (8 * B + 255) // 256 * 256
    m_tiles = (q_len * heads + M_TILE - 1) // M_TILE
    nu = units_max(B, m_tiles, max_pages, num_splits)
    work = ws[woff:woff + 32 * nu].view(np.int32).reshape(nu, 8)
    return req, work, m_tiles


def check(seq_lens, heads, q_len, max_pages, num_splits, what):
    say(f"plan {what}: B={len(seq_lens)} H={heads} q_len={q_len} max_pages={max_pages} splits={num_splits}")
    req, work, m_tiles = run_plan(seq_lens, heads, q_len, max_pages, num_splits)
    target = min(torch.cuda.get_device_properties(0).multi_processor_count, TARGET_CAP)
    S, first, units = expected_plan(seq_lens, max_pages, m_tiles, num_splits, target)
    np.testing.assert_array_equal(req[:, 0], S, err_msg=f"{what}: splits per request")
    np.testing.assert_array_equal(req[:, 1], first, err_msg=f"{what}: first kv-unit")
    K = len(units)
    assert work.shape[0] >= ((K + 7) // 8) * 8 * m_tiles, f"{what}: work list too short"
    C = (K + 7) // 8
    seen = set()
    for u in range(work.shape[0]):
        kx, mt = divmod(u // 8, m_tiles)
        k = C * (u % 8) + kx
        w = work[u]
        if kx >= C or k >= K:
            assert w[0] == -1, f"{what}: slot {u} should be empty, holds {w.tolist()}"
            continue
        b, s, pb, pe, ns = units[k]
        seen.add((k, mt))
        assert w.tolist() == [b, mt, s, pb, pe, ns, 0, 0], \
            f"{what}: slot {u} (kv-unit {k}, tile {mt}) = {w.tolist()}, expected {[b, mt, s, pb, pe, ns, 0, 0]}"
    assert len(seen) == K * m_tiles, f"{what}: {K * m_tiles - len(seen)} (kv-unit, tile) pairs have no slot"
    return S


def ragged(B, lo, hi, seed, zeros=0):
    rng = np.random.default_rng(seed)
    s = rng.integers(lo, hi + 1, size=B)
    if zeros:
        s[rng.choice(B, size=zeros, replace=False)] = 0
    return s.tolist()


def test_plan_uniform_batch64_h128():
    """The batch 64, 128 head, 4096 token shape: the answer is one of the first candidates."""
    check([4096] * 64, 128, 1, 64, 0, "uniform")


def test_plan_ragged_two_tiles():
    """Ragged lengths, q_len 2 x 96 heads (two row tiles), some empty requests."""
    check(ragged(37, 1, 20000, 11, zeros=3), 96, 2, 313, 0, "ragged two tiles")


def test_plan_one_long_request_bisects():
    """One long request among short ones: the first 16 candidates do not fit, so
    the planner searches the rest of the range (16 spread candidates a round)."""
    S = check([64] * 199 + [100000], 16, 1, 1563, 0, "one long request")
    assert S[-1] > 1 and (S[:-1] == 1).all()


def test_plan_more_requests_than_units():
    """More requests than workgroups of one round: every request gets one split
    (threads hold several requests each)."""
    S = check(ragged(3000, 0, 700, 12, zeros=50), 16, 1, 11, 0, "batch 3000")
    assert (S == 1).all()


def test_plan_past_lds_cache():
    """More requests than the planner caches in LDS (8192): the rest are read from HBM."""
    check(ragged(9000, 1, 128, 13), 16, 1, 2, 0, "batch 9000")


def test_plan_fixed_splits():
    """num_splits = 3 with requests shorter than 3 pages and empty ones."""
    check(ragged(50, 0, 600, 14, zeros=5), 32, 1, 10, 3, "fixed 3 splits")


@pytest.mark.parametrize("batch", [256, 257])
def test_plan_threshold_between_fused_and_planner_kernel(batch):
    """256 requests are planned inside the decode kernel, 257 by the planner
    kernel: both give the policy's split list."""
    check(ragged(batch, 0, 5000, 15 + batch, zeros=7), 16, 1, 79, 0, f"batch {batch}")
