"""The device planner's work list, checked integer for integer.

The planner (one workgroup, no host sync) reads seq_lens on the device and
writes, into the workspace, per request its piece count, first piece and first
global page, and the list of work items the decode kernel runs.  Which list it
picks only moves time around, so an error in it would show up as lost speed,
not as a parity failure; this test reads the list back and compares it with
the policy restated below in plain Python:

* a request of n cache tokens has P = ceil(n / 64) pages;
* num_splits = k > 0: max(1, min(k, P)) splits of ceil(P / S) pages;
* automatic: the smallest chunk c (pages) with c >= max(2, ceil(sum P / U))
  such that sum_b max(1, ceil(P_b / c)) <= U, where U = max(1, target // m_tiles)
  and target = min(compute units, 256); if no chunk up to the longest request
  fits, every request gets one split;
* split s of request b covers pages [min(P, s c), min(P, (s + 1) c)); kv-units
  are numbered request by request, split by split (K in all), and kv-unit k is
  piece k;
* balanced (fp8 caches only, automatic splits): when c > A + max(1, A // 8),
  A = max(2, ceil(sum P / U)), the common chunk fits (sum max(1, ceil(P_b / c))
  <= U), and A + 2 X + max(1, A // 8) < c, X the most requests that start
  strictly inside one kv-unit below, all requests' pages are laid end to end (request
  b starts at global page G_b) and kv-unit k covers the global pages
  [k A, min((k + 1) A, sum P)) (K = ceil(sum P / A)); request b is cut into one
  piece per kv-unit it touches (none when empty), pieces numbered request by
  request; a kv-unit's work item names the request holding its first page,
  the local page there, its page count, and that request's first piece in the
  kv-unit and piece count;
* with C = ceil(K / 8), work slot u holds kv-unit k = C (u % 8) + (u // 8) // m_tiles
  and row tile (u // 8) % m_tiles, or is empty when (u // 8) // m_tiles >= C or
  k >= K (the XCD-contiguous order: slot u runs on XCD u % 8).

The workspace layout read here is the library's internal one: int32 [B][4]
(pieces, first piece, first global page or 0, 0) at offset 0, then 32-byte
work items (b, mt, piece, page_begin, npages, nsplit, g0, chunk) at the next
256-byte boundary (an empty slot: b = -1 and zeros).
"""
import numpy as np
import pytest
import torch

from tests.gpu_common import say

pytestmark = pytest.mark.gpu

PAGE = 64
MIN_CHUNK = 2
TARGET_CAP = 256
PIECE_COST = 2
M_TILE = 128


def pages_of(seq_lens, max_pages):
    n = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, max_pages * PAGE)
    return (n + PAGE - 1) // PAGE


def expected_plan(seq_lens, max_pages, m_tiles, num_splits, target, fp8=False):
    """(req_info rows, work items) of the policy above; an item is
    (b, piece, page_begin, npages, nsplit, g0, chunk) without the row tile
    (one per kv-unit, or per group of splits)."""
    pg = pages_of(seq_lens, max_pages)
    B = len(pg)
    cap = max(1, target // m_tiles)
    if num_splits > 0:
        S = np.maximum(1, np.minimum(num_splits, pg))
        cb = (pg + S - 1) // S
        chunk = None
        # groups of consecutive splits (bf16 two-role kernel, forced splits
        # making more items than one round): when every request has the same
        # split count S, the smallest divisor g of S that brings the items
        # within the round; an item is then g splits of one request
        per_req = min(num_splits, max_pages)
        group_ok = not fp8 and per_req > 1 and B * per_req * m_tiles > target
        S_all = min(num_splits, max(1, int(pg.max())))
        K = int(S.sum())
        if group_ok and K == B * S_all and K * m_tiles > target:
            need = min(-(-K * m_tiles // target), S_all)
            g = next(d for d in range(need, S_all + 1) if S_all % d == 0)
            if g > 1:
                first = np.concatenate([[0], np.cumsum(S)[:-1]])
                req = np.stack([S, first, np.zeros(B, dtype=np.int64), np.zeros(B, dtype=np.int64)], axis=1)
                items = []
                for b in range(B):
                    for s0 in range(0, int(S[b]), g):
                        pb, pe = min(pg[b], s0 * cb[b]), min(pg[b], (s0 + g) * cb[b])
                        items.append((b, int(first[b] + s0), int(pb), int(pe - pb), int(S[b]), g, 0))
                return req, items
    else:
        start = max(MIN_CHUNK, -(-int(pg.sum()) // cap))
        longest = max(1, int(pg.max()))
        chunk = None
        for c in range(start, longest + 1):
            if int(np.maximum(1, (pg + c - 1) // c).sum()) <= cap:
                chunk = c
                break
        if chunk is None:
            chunk = max(start, longest)
        A = max(MIN_CHUNK, -(-int(pg.sum()) // cap))
        T = int(pg.sum())
        G = np.concatenate([[0], np.cumsum(pg)[:-1]])
        balanced = (fp8 and 0 < T < 2 ** 30 and chunk > A + max(1, A // 8)
                    and int(np.maximum(1, (pg + chunk - 1) // chunk).sum()) <= cap)
        if balanced:
            # every piece costs PIECE_COST pages besides its own: the busiest
            # kv-unit (one piece more per request starting inside it) must
            # still beat the common chunk by 1/8
            inside = np.zeros(-(-T // A), dtype=np.int64)
            for b in np.nonzero((pg > 0) & (G % A != 0))[0]:
                inside[G[b] // A] += 1
            balanced = A + PIECE_COST * int(inside.max()) + max(1, A // 8) < chunk
        if balanced:
            n = np.where(pg > 0, (G + pg - 1) // A - G // A + 1, 0)
            first = np.concatenate([[0], np.cumsum(n)[:-1]])
            req = np.stack([n, first, G, np.zeros(B, dtype=np.int64)], axis=1)
            K = -(-T // A)
            items = []
            for k in range(K):
                g0 = k * A
                b = int(np.nonzero((G <= g0) & (g0 < G + pg))[0][0])
                items.append((b, int(first[b] + k - G[b] // A), g0 - int(G[b]), min(g0 + A, T) - g0,
                              int(n[b]), g0, A))
            return req, items
        S = np.maximum(1, (pg + chunk - 1) // chunk)
        cb = np.full(B, chunk, dtype=np.int64)
    first = np.concatenate([[0], np.cumsum(S)[:-1]])
    req = np.stack([S, first, np.zeros(B, dtype=np.int64), np.zeros(B, dtype=np.int64)], axis=1)
    items = []
    for b in range(B):
        for s in range(int(S[b])):
            pb, pe = min(pg[b], s * cb[b]), min(pg[b], (s + 1) * cb[b])
            items.append((b, len(items), int(pb), int(pe - pb), int(S[b]), 0, 0))
    return req, items


def units_max(B, m_tiles, max_pages, num_splits):
    if num_splits > 0:
        k = B * max(1, min(num_splits, max_pages))
    else:
        k = TARGET_CAP // m_tiles + B
    return ((k + 7) // 8) * 8 * m_tiles


def run_plan(seq_lens, heads, q_len, max_pages, num_splits, fp8=False, planned=False):
    import mla_latent_decode_absorbed_amd as mla
    dev = torch.device("cuda:0")
    B = len(seq_lens)
    pool = 4
    g = torch.Generator().manual_seed(1234 + B)
    if fp8:
        q = (torch.randn((B, q_len, heads, 576), generator=g) * 0.5).to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
        kv = (torch.randn((pool, PAGE, 576), generator=g) * 0.5).to(torch.float8_e4m3fn).view(torch.uint8).to(dev)
        kv_scale = torch.tensor([1.0], dtype=torch.float32, device=dev)
    else:
        q = (torch.randn((B, q_len, heads, 576), generator=g) * 0.5).to(torch.bfloat16).to(dev)
        kv = (torch.randn((pool, PAGE, 576), generator=g) * 0.5).to(torch.bfloat16).to(dev)
        kv_scale = None
    bt = torch.randint(0, pool, (B, max_pages), generator=g, dtype=torch.int32).to(dev)
    sl = torch.tensor(seq_lens, dtype=torch.int32).to(dev)
    desc = mla.make_desc(B, q_len, heads, pool, max_pages, num_splits=num_splits,
                         kv_dtype=mla.FP8_E4M3 if fp8 else mla.BF16)
    dec = mla.Decoder(desc, device=dev)
    dec.workspace.fill_(0xAB)
    if planned:
        # the planner kernel (one workgroup) builds the list, whatever the batch
        dec.plan(sl)
        out, lse = dec.planned(q, kv, bt, sl, 0.07, kv_scale=kv_scale)
    else:
        out, lse = dec(q, kv, bt, sl, 0.07, kv_scale=kv_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ws = dec.workspace.cpu().numpy()
    req = ws[:16 * B].view(np.int32).reshape(B, 4)
    woff = (16 * B + 255) // 256 * 256
    m_tiles = (q_len * heads + M_TILE - 1) // M_TILE
    nu = units_max(B, m_tiles, max_pages, num_splits)
    work = ws[woff:woff + 32 * nu].view(np.int32).reshape(nu, 8)
    return req, work, m_tiles


def check(seq_lens, heads, q_len, max_pages, num_splits, what, fp8=False, planned=False):
    say(f"plan {what}: B={len(seq_lens)} H={heads} q_len={q_len} max_pages={max_pages} splits={num_splits} "
        f"{'fp8' if fp8 else 'bf16'}{' planner kernel' if planned else ''}")
    req, work, m_tiles = run_plan(seq_lens, heads, q_len, max_pages, num_splits, fp8, planned)
    target = min(torch.cuda.get_device_properties(0).multi_processor_count, TARGET_CAP)
    req_exp, items = expected_plan(seq_lens, max_pages, m_tiles, num_splits, target, fp8)
    np.testing.assert_array_equal(req, req_exp, err_msg=f"{what}: per-request (pieces, first piece, first page)")
    K = len(items)
    assert work.shape[0] >= ((K + 7) // 8) * 8 * m_tiles, f"{what}: work list too short"
    C = (K + 7) // 8
    seen = set()
    for u in range(work.shape[0]):
        kx, mt = divmod(u // 8, m_tiles)
        k = C * (u % 8) + kx
        w = work[u].tolist()
        if kx >= C or k >= K:
            assert w == [-1, 0, 0, 0, 0, 0, 0, 0], f"{what}: slot {u} should be empty, holds {w}"
            continue
        b, piece, pb, npg, ns, g0, chunk = items[k]
        seen.add((k, mt))
        exp = [b, mt, piece, pb, npg, ns, g0, chunk]
        assert w == exp, f"{what}: slot {u} (kv-unit {k}, tile {mt}) = {w}, expected {exp}"
    assert len(seen) == K * m_tiles, f"{what}: {K * m_tiles - len(seen)} (kv-unit, tile) pairs have no slot"
    return req[:, 0], req_exp


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
    S, _ = check([64] * 199 + [100000], 16, 1, 1563, 0, "one long request")
    assert S[-1] > 1 and (S[:-1] == 1).all()


def test_plan_more_requests_than_units():
    """More requests than workgroups of one round: every request gets one split
    (threads hold several requests each)."""
    S, _ = check(ragged(3000, 0, 700, 12, zeros=50), 16, 1, 11, 0, "batch 3000")
    assert (S == 1).all()


def test_plan_past_lds_cache():
    """More requests than the planner caches in LDS (8192): the rest are read from HBM."""
    check(ragged(9000, 1, 128, 13), 16, 1, 2, 0, "batch 9000")


def test_plan_fixed_splits():
    """num_splits = 3 with requests shorter than 3 pages and empty ones."""
    check(ragged(50, 0, 600, 14, zeros=5), 32, 1, 10, 3, "fixed 3 splits")


@pytest.mark.parametrize("planned", [False, True])
def test_plan_fixed_splits_grouped(planned):
    """256 splits of 4 x 131072 tokens over two row tiles (2048 kv-units x
    tiles): groups of 8 consecutive splits, one round of 256 workgroups."""
    req, _ = check([131072] * 4, 128, 2, 2048, 256, "256 splits grouped", planned=planned)
    assert (req == 256).all()


def test_plan_fixed_splits_group_is_a_divisor():
    """9 splits x 40 requests (360 items): the group is 3, the smallest divisor
    of 9 at or above 2; and one short request (fewer splits) turns grouping off."""
    check([9 * 64 * 3] * 40, 64, 1, 27, 9, "9 splits grouped by 3")
    check([9 * 64 * 3] * 39 + [64 * 5], 64, 1, 27, 9, "unequal split counts: no groups")


@pytest.mark.parametrize("batch", [256, 257])
def test_plan_threshold_between_fused_and_planner_kernel(batch):
    """256 requests are planned inside the decode kernel, 257 by the planner
    kernel: both give the policy's split list."""
    check(ragged(batch, 0, 5000, 15 + batch, zeros=7), 16, 1, 79, 0, f"batch {batch}")


def test_plan_balanced_fp8_ragged_batch128():
    """The ragged fp8 shape (128 requests of 1k-16k tokens, 128 heads): the
    common chunk leaves the longest kv-unit well above the average, so the
    balanced plan is taken (some request starts past global page 0)."""
    lens = ragged(128, 1024, 16384, 21)
    _, req = check(lens, 128, 1, 256, 0, "balanced ragged 128", fp8=True)
    assert (req[:, 2] > 0).any(), "expected the balanced plan"


def test_plan_balanced_two_tiles_empty_and_short():
    """Balanced plan with two row tiles, empty requests (no piece) and short ones."""
    lens = ragged(40, 100, 30000, 22, zeros=4)
    lens[5] = 65
    lens[6] = 1
    check(lens, 96, 2, 469, 0, "balanced two tiles", fp8=True)


def test_plan_balanced_by_the_planner_kernel():
    """The same ragged fp8 batch planned by the planner kernel (the plan/reuse
    entry points): the balanced list again, from the other copy of the planner."""
    lens = ragged(128, 1024, 16384, 21)
    _, req = check(lens, 128, 1, 256, 0, "balanced ragged 128", fp8=True, planned=True)
    assert (req[:, 2] > 0).any(), "expected the balanced plan"


def test_plan_fp8_more_requests_than_units():
    """300 ragged fp8 requests (more than one round of workgroups): the common
    chunk (one split each), from the planner kernel."""
    check(ragged(300, 200, 20000, 23, zeros=3), 16, 1, 313, 0, "fp8 batch 300", fp8=True)


def test_plan_fp8_uniform_keeps_common_chunk():
    """Equal lengths: the common chunk is already balanced, and stays."""
    _, req = check([4096] * 64, 128, 1, 64, 0, "fp8 uniform", fp8=True)
    assert (req[:, 2] == 0).all()


def test_plan_fp8_one_long_request_among_tiny():
    """One long request among 199 one-page ones on an fp8 cache: kv-units of the
    balanced plan would hold many one-page pieces; the policy weighs their
    fixed cost against the common chunk's longest unit."""
    check([64] * 199 + [100000], 16, 1, 1563, 0, "fp8 one long request", fp8=True)


def test_plan_balanced_lengths_of_the_parity_test():
    """The lengths the balanced-plan parity test uses do take the balanced plan."""
    from tests.gpu_common import balanced_plan_lens
    _, req = check(balanced_plan_lens(), 16, 1, 64, 0, "parity-test lengths", fp8=True)
    assert (req[:, 2] > 0).any()
