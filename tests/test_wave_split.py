"""The decode plan's wave split, modelled on the host (no GPU): for any mix of pair sizes,
share sizes and worker counts, the shares it cuts are non-empty, consecutive, cover every
block once, and each begins inside the pair its unit record names.  This is the property
the decode and merge kernels rely on (a cut pair's contributors are the consecutive waves
whose shares start before its end); the model follows the arithmetic of the plan kernel
(csrc/plan.hip): weights 4 nb + C per pair, W = ceil(T / min_blocks) capped at the worker
count and, below it and above one workgroup per compute unit, rounded down to whole such
rounds, the effective
pair cost C' = C while 4 T / W >= C + 5 (else 4 T / W - 5, at least 0), and share w starting
at weighted position floor(w TW / W).  The plan also counts, per share, the shares that the
cut pair opened by its last segment spans (the merge task's contributors); the model checks
that count against the shares that meet each pair, found by brute force."""
import numpy as np
import pytest


def plan_split(nbs, heads, min_blocks, max_waves, pair_cost, wave_round=0):
    """Share starts wx0[0..W] and the unit of each share, as the plan kernel computes them.
    nbs: blocks per decode unit (row); each unit has `heads` pairs of that size."""
    nbs = np.asarray(nbs, np.int64)
    H = heads
    T = int(nbs.sum()) * H
    NP = int((nbs > 0).sum()) * H
    if T == 0:
        return [0], []
    W = (T + min_blocks - 1) // min_blocks
    W = max(1, min(W, max_waves))
    if W < max_waves and wave_round > 0 and W > wave_round:
        W = W // wave_round * wave_round
    room = 4 * T // W
    C = pair_cost
    if W > 1:
        C = C if room >= C + 5 else (room - 5 if room > 5 else 0)
    TW = 4 * T + C * NP
    cb = np.concatenate([[0], np.cumsum(nbs * H)])
    cw = np.concatenate([[0], np.cumsum(np.where(nbs > 0, (4 * nbs + C) * H, 0))])
    assert cw[-1] == TW
    wx0 = [None] * (W + 1)
    wu = [None] * W
    for u in range(len(nbs)):
        c0, c1 = int(cw[u]), int(cw[u + 1])
        if c1 == c0:
            continue
        w0 = (c0 * W + TW - 1) // TW
        w1 = min((c1 * W + TW - 1) // TW, W)
        nb = int(nbs[u])
        pw = 4 * nb + C
        for w in range(w0, w1):
            y = (w * TW) // W - c0
            g, o = divmod(y, pw)
            k = 0 if o <= C else (o - C + 3) // 4
            k = min(k, nb)
            wx0[w] = int(cb[u]) + g * nb + k
            wu[w] = u
    wx0[W] = T
    assert all(x is not None for x in wx0), "a share start was not written"
    return wx0, wu


def plan_cut_counts(nbs, heads, wx0, wu):
    """Per share, the plan's count of the shares that the cut pair opened by its last
    segment spans (0: no such pair): the pair holding the share's last block is cut when it
    starts inside the share and ends past it; its count is the number of shares that start
    before its end, found by a binary search over the later share starts (csrc/plan.hip)."""
    nbs = np.asarray(nbs, np.int64)
    cb = np.concatenate([[0], np.cumsum(nbs * heads)])
    W = len(wu)
    out = []
    for w in range(W):
        x0, x1 = wx0[w], wx0[w + 1]
        u = wu[w]
        while cb[u + 1] <= x0:
            u += 1
        ul = u
        while cb[ul + 1] <= x1 - 1:
            ul += 1
        nb = int(nbs[ul])
        psl = int(cb[ul]) + (x1 - 1 - int(cb[ul])) // nb * nb
        pel = psl + nb
        nc = 0
        if psl >= x0 and pel > x1:
            lo, hi = w + 1, W
            while lo < hi:
                mid = (lo + hi) // 2
                if wx0[mid] < pel:
                    lo = mid + 1
                else:
                    hi = mid
            nc = lo - w
        out.append(nc)
    return out


def brute_cut_counts(nbs, heads, wx0):
    """The same by definition: every pair, the shares whose block ranges meet it; a pair met
    by several shares is counted at the share holding its first block."""
    nbs = np.asarray(nbs, np.int64)
    W = len(wx0) - 1
    out = [0] * W
    pos = 0
    for nb in nbs.tolist():
        for _ in range(heads):
            ps, pe = pos, pos + nb
            pos = pe
            if nb == 0:
                continue
            meet = [w for w in range(W) if wx0[w] < pe and wx0[w + 1] > ps]
            if len(meet) > 1:
                assert wx0[meet[0]] <= ps < wx0[meet[0] + 1]   # the first holds its start
                out[meet[0]] = len(meet)
    return out


def check(nbs, heads, min_blocks, max_waves, pair_cost, wave_round=0):
    wx0, wu = plan_split(nbs, heads, min_blocks, max_waves, pair_cost, wave_round)
    if wu:
        assert plan_cut_counts(nbs, heads, wx0, wu) == brute_cut_counts(nbs, heads, wx0), (
            nbs, heads, min_blocks, max_waves, pair_cost, wave_round)
    T = int(np.sum(nbs)) * heads
    assert wx0[0] == 0 and wx0[-1] == T
    # non-empty and consecutive: strictly increasing starts cover [0, T)
    assert all(b > a for a, b in zip(wx0, wx0[1:])), (nbs, heads, min_blocks, max_waves)
    # each share starts inside the unit it names (or at the unit's end, i.e. the next
    # pair's first block of the same unit: a start is never before the unit)
    cb = np.concatenate([[0], np.cumsum(np.asarray(nbs) * heads)])
    for w, u in enumerate(wu):
        assert cb[u] <= wx0[w] < cb[u + 1] or wx0[w] == cb[u + 1], (w, u)


@pytest.mark.parametrize("min_blocks", [4, 5, 8, 16, 33])
@pytest.mark.parametrize("pair_cost", [0, 14, 22, 27])
def test_shares_nonempty_random(min_blocks, pair_cost):
    rng = np.random.default_rng(1000 * min_blocks + pair_cost)
    for _ in range(60):
        n = int(rng.integers(1, 40))
        kind = rng.integers(0, 3)
        if kind == 0:
            nbs = rng.integers(0, 6, size=n)                  # many tiny pairs
        elif kind == 1:
            nbs = rng.integers(1, 300, size=n)
        else:
            nbs = np.rint(np.exp(rng.normal(3, 1.5, size=n))).astype(int)   # log-normal
        heads = int(rng.choice([1, 2, 4, 8]))
        max_waves = int(rng.choice([1, 3, 17, 64, 1024, 4096]))
        wave_round = int(rng.choice([0, 4, 12, 64]))
        check(nbs, heads, min_blocks, max_waves, pair_cost, wave_round)


def test_shares_edge_cases():
    check([1], 1, 16, 4096, 27)            # one block
    check([0, 0, 3], 1, 4, 4096, 27)       # empty units
    check([16], 1, 16, 4096, 27)           # exactly one share's worth
    check([17], 1, 16, 4096, 27)           # T / W = 8.5, the tightest case at 16
    check([5], 1, 4, 4096, 27)             # T / W = 2.5 at the 4-block floor
    check([1] * 50, 8, 4, 4096, 27)        # only one-block pairs
    check([100000], 8, 16, 4096, 27)       # capped by the worker count
    check([8312], 1, 12, 2048, 14, 1024)   # below one round: 693 shares, unrounded
    check([8312], 1, 8, 2048, 14, 1024)    # 1039 shares rounded down to 1024
    check([5000], 1, 4, 2048, 14, 1024)    # 1250 rounded to 1024: shares of 4.9 blocks


def test_whole_rounds():
    # the worker counts the rule gives: capped, unrounded below a round, whole rounds above
    assert len(plan_split([100000], 8, 12, 4096, 14, 1024)[1]) == 4096
    assert len(plan_split([8312], 1, 12, 2048, 14, 1024)[1]) == 693
    assert len(plan_split([8312], 1, 8, 2048, 14, 1024)[1]) == 1024
    assert len(plan_split([30000], 1, 12, 4096, 14, 1024)[1]) == 2048


def test_effective_cost_is_needed():
    """Without lowering the pair cost, small shares would come out empty: the model with the
    unlowered cost must fail on a case the plan handles (a check that the test can fail)."""
    nbs, heads, mb = [5], 1, 4
    T = 5
    W = 2
    C = 27
    TW = 4 * T + C
    starts = [(w * TW) // W for w in range(W)]
    ks = [0 if s <= C else (s - C + 3) // 4 for s in starts]
    assert ks[0] == ks[1]            # both shares would start at block 0
    check(nbs, heads, mb, 4096, C)   # the plan's rule keeps them apart
