"""fa_fwd_ex's host-side work plan (fa_fwd_schedule; no device involved).

Every query tile must be covered exactly once: its nominal key blocks
(ceil(min(Nk, 128 (t+1) + Nk - Nq) / bn) under the causal mask, the queries
being the last Nq of Nk positions; ceil(Nk / bn) without; bn, the keys per
block, as the header documents) are partitioned by the parts of the tile,
split tiles own disjoint
partial-state slots, and the items come longest first under the planner's
stated cost model. The schedule simulation that chose the plan is
re-implemented here from its description (compute units of `occ` slots whose
throughput depends on how many workgroups are resident; a freed slot takes
the next workgroup in dispatch order), and the chosen plan must shorten it by
the planner's required margin.
"""
import heapq
import math

import pytest

from exact_io_aware_17_amd import _lib

BM = 128


def block_keys(d, Nq, Nk, BH, causal, cus):
    """Keys per block of the forward launch (the header's rule: 64 keys)."""
    return 64
ITEM, SPLIT = 2.0, 7.0   # cost per item and extra per split part, in key blocks
MIN_GAIN = 0.75


def tile_blocks(N, t, causal, Nk=None, bn=32):
    Nk = N if Nk is None else Nk
    kend = max(0, min(Nk, BM * (t + 1) + Nk - N)) if causal else Nk
    return math.ceil(kend / bn)


def decode(item):
    return item & 0xFFF, (item >> 12) & 15, ((item >> 16) & 15) + 1, item >> 20


def cu_throughput(k, occ):
    return 1.0 if k >= occ else min(1.0, 0.40 + 0.35 * (k - 1))


def simulate(costs, BH, cus, occ):
    total, nxt = len(costs) * BH, 0
    rem = [[] for _ in range(cus)]
    tt = [0.0] * cus

    def rate(c):
        k = len(rem[c])
        return cu_throughput(k, occ) * occ / k if k else 0.0

    ev = []

    def sched(c):
        if rem[c]:
            heapq.heappush(ev, (tt[c] + min(rem[c]) / rate(c), c))

    for _ in range(occ):
        for c in range(cus):
            if nxt < total:
                rem[c].append(costs[nxt // BH])
                nxt += 1
    for c in range(cus):
        sched(c)
    end = 0.0
    while ev:
        t, c = heapq.heappop(ev)
        if not rem[c]:
            continue
        mn = min(rem[c])
        if abs(tt[c] + mn / rate(c) - t) > 1e-9 * (1 + t):
            continue
        rem[c] = [r - mn for r in rem[c] if r - mn > 1e-12]
        tt[c] = t
        end = max(end, t)
        while len(rem[c]) < occ and nxt < total:
            rem[c].append(costs[nxt // BH])
            nxt += 1
        sched(c)
    return end


# (Nq, Nk, BH, causal, cus, occ[, d])
CASES = [
    (4096, 4096, 32, True, 256, 3),     # the metric shape: several waves of work, not split
    (4096, 4096, 32, False, 256, 3),
    (16384, 16384, 2, True, 256, 3),    # few heads, long rows: split
    (16384, 16384, 1, False, 256, 3),
    (8192, 8192, 4, True, 256, 3),
    (1000, 1000, 6, True, 256, 3),      # ragged last tile
    (1024, 1024, 1, False, 256, 3),
    (640, 640, 4, False, 256, 5),
    (64, 64, 1, True, 256, 3),
    (4096, 4096, 32, True, 0, 0),       # unknown device: never split
    (65536, 65536, 64, True, 256, 3),   # many waves of work: never split
    (1, 32768, 32, True, 256, 3),       # one decode query per head over a long cache
    (16, 8192, 8, False, 256, 3),
    (1024, 8192, 4, True, 256, 3),      # a continuation after a 7168-key prefix
    (2048, 1000, 2, True, 256, 3),      # Nq > Nk: early query tiles see no key
    (16384, 16384, 2, True, 256, 3, 64),  # 64-key blocks (d <= 64)
    (4096, 4096, 4, False, 256, 3, 32),
    (1, 32768, 8, True, 256, 3, 64),
]
CASES = [c if len(c) == 7 else c + (128,) for c in CASES]


def _costs(items, N, Nk, causal, bn):
    out = []
    for it in items:
        t, part, np_, _ = decode(it)
        nb = tile_blocks(N, t, causal, Nk, bn)
        out.append((part + 1) * nb // np_ - part * nb // np_ + ITEM + (SPLIT if np_ > 1 else 0))
    return out


@pytest.mark.parametrize("N,Nk,BH,causal,cus,occ,d", CASES)
def test_plan_covers_every_tile_once(N, Nk, BH, causal, cus, occ, d):
    items, nslots = _lib.schedule(N, BH, causal, cus, occ, Nk, d)
    bn = block_keys(d, N, Nk, BH, causal, cus)
    ntiles = math.ceil(N / BM)
    if not items:
        return
    assert len(items) <= 512
    parts = {}
    for it in items:
        t, part, np_, sb = decode(it)
        assert 0 <= t < ntiles
        assert part < np_
        parts.setdefault(t, []).append((part, np_, sb))
    assert sorted(parts) == list(range(ntiles))
    used = set()
    for t, ps in parts.items():
        np_ = ps[0][1]
        assert sorted(p for p, _, _ in ps) == list(range(np_))
        assert all(n == np_ for _, n, _ in ps)
        nb = tile_blocks(N, t, causal, Nk, bn)
        ranges = sorted((p * nb // np_, (p + 1) * nb // np_) for p, _, _ in ps)
        assert ranges[0][0] == 0 and ranges[-1][1] == nb
        assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
        if np_ > 1:
            assert all(lo < hi for lo, hi in ranges)  # no empty nominal part
            sb = ps[0][2]
            assert all(s == sb for _, _, s in ps)
            slots_t = set(range(sb, sb + np_))
            assert not (slots_t & used)
            used |= slots_t
            assert sb + np_ <= nslots


@pytest.mark.parametrize("N,Nk,BH,causal,cus,occ,d", CASES)
def test_plan_is_longest_first_and_pays_off(N, Nk, BH, causal, cus, occ, d):
    items, _ = _lib.schedule(N, BH, causal, cus, occ, Nk, d)
    if not items:
        return
    bn = block_keys(d, N, Nk, BH, causal, cus)
    costs = _costs(items, N, Nk, causal, bn)
    assert all(a >= b for a, b in zip(costs, costs[1:]))
    ntiles = math.ceil(N / BM)
    unsplit = sorted((tile_blocks(N, t, causal, Nk, bn) + ITEM for t in range(ntiles)),
                     reverse=True)
    assert simulate(costs, BH, cus, occ) < MIN_GAIN * simulate(unsplit, BH, cus, occ)


def test_split_only_underfilled_grids():
    assert _lib.schedule(4096, 32, True, 256, 3) == ([], 0)    # metric shape: one item per tile
    items, nslots = _lib.schedule(16384, 2, True, 256, 3)
    assert len(items) > 128 and nslots > 0
    assert _lib.schedule(16384, 2, True, 256, 3) == (items, nslots)  # cached, deterministic
    assert max(decode(it)[2] for it in _lib.schedule(1024, 1, False, 256, 3)[0]) == 4
    # Decode (one query per head) over a long cache: every head's only tile
    # split, here into the most parts an item can have.
    items, nslots = _lib.schedule(1, 32, True, 256, 3, 32768)
    assert len(items) == 16 and nslots == 16
    assert sorted(decode(it)[1] for it in items) == list(range(16))
    assert all(decode(it)[2] == 16 and decode(it)[3] == 0 for it in items)
    assert _lib.schedule(1, 32, True, 256, 3, 32768) != _lib.schedule(1, 32, True, 256, 3, 1)


def test_schedule_argument_errors():
    lib = _lib.load()
    INV = _lib.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_schedule(0, 128, 1, 128, 1, 256, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 0, 1, 128, 1, 256, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 0, 128, 1, 256, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 1, 0, 1, 256, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 1, 128, 5, 256, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 1, 128, 1, -1, 3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 1, 128, 1, 256, -3, None, 0, None) == INV
    assert lib.fa_fwd_schedule(128, 128, 1, 128, 1, 256, 3, None, 4, None) == INV
