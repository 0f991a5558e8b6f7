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
import os
import math

import pytest

from exact_io_aware_17_amd import _lib

BM = 128


def block_keys(d, Nq, Nk, BH, causal, cus):
    """Keys per block of the forward launch (the header's rule: 64 keys)."""
    return 64
ITEM, SPLIT = 2.0, 7.0   # cost per item and extra per split part, in key blocks
MERGE = 0.15             # extra per split part for each part of its tile beyond 16 (the merge)
MIN_GAIN = 0.75


def tile_blocks(N, t, causal, Nk=None, bn=32):
    Nk = N if Nk is None else Nk
    kend = max(0, min(Nk, BM * (t + 1) + Nk - N)) if causal else Nk
    return math.ceil(kend / bn)


def decode(item):
    """tile | part << 9 | (nparts - 1) << 15 | slot_base << 21 (the header's layout)."""
    return item & 0x1FF, (item >> 9) & 63, ((item >> 15) & 63) + 1, item >> 21


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
        out.append((part + 1) * nb // np_ - part * nb // np_ + ITEM
                   + (SPLIT + MERGE * max(0, np_ - 16) if np_ > 1 else 0))
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
    # split, into more parts than a multi-tile plan may use (at most 64).
    for BH, Nk in ((32, 32768), (8, 131072), (8, 32768)):
        items, nslots = _lib.schedule(1, BH, True, 256, 3, Nk)
        P = len(items)
        assert 16 < P <= 64 and nslots == P
        assert sorted(decode(it)[1] for it in items) == list(range(P))
        assert all(decode(it)[0] == 0 and decode(it)[2] == P and decode(it)[3] == 0 for it in items)
    # Several tiles: never more than 16 parts per tile.
    for args in ((16384, 2, True, 256, 3), (1024, 1, False, 256, 3), (2048, 1, True, 256, 2, 65536)):
        assert max(decode(it)[2] for it in _lib.schedule(*args)[0]) <= 16
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


def _rss_bytes():
    with open("/proc/self/statm") as f:
        return int(f.read().split()[1]) * os.sysconf("SC_PAGE_SIZE")


def test_plan_cache_stays_bounded_over_a_decode_loop():
    """A decode loop plans one more key per step: 20,000 consecutive key
    counts (313 distinct block counts, more than the cache holds) must not
    grow the host memory by a plan per step (about 2 KiB each, 40 MB in
    all), and key counts with the same block count share one plan."""
    import ctypes
    lib = _lib.load()
    buf = (ctypes.c_uint32 * 4096)()
    ns = ctypes.c_int(0)
    lib.fa_fwd_schedule(1, 1, 64, 128, 1, 256, 2, buf, 4096, ctypes.byref(ns))
    r0 = _rss_bytes()
    for nk in range(1, 20001):
        n = lib.fa_fwd_schedule(1, nk, 64, 128, 1, 256, 2, buf, 4096, ctypes.byref(ns))
        assert n >= 0
    assert _rss_bytes() - r0 < 8 * 2 ** 20
    a = _lib.schedule(1, 64, True, 256, 2, Nk=4097, d=128)
    b = _lib.schedule(1, 64, True, 256, 2, Nk=4160, d=128)   # same 65 blocks of 64 keys
    c = _lib.schedule(1, 64, True, 256, 2, Nk=4161, d=128)   # 66 blocks
    assert a == b
    assert a[0] and c[0]


# ---- tile order (fa_fwd_tile_order; host only with explicit cus, occ) ----

L2_BYTES = 4 << 20   # one XCD's L2 cache, the header's threshold


def expected_order(Nq, Nk, BH, d, causal, cus, occ):
    """The header's rule: pairs under a causal mask when one head's K and V
    (2 * Nk * d two-byte elements) are at least one XCD's L2 and the pairs
    still fill every resident slot; else heads one after another per XCD when
    B*H is a multiple of 8 and the grid is at least 16 rounds of slots."""
    ntiles = -(-Nq // BM)
    paired = (causal and ntiles >= 2 and 2 * Nk * d * 2 >= L2_BYTES
              and BH * (-(-ntiles // 2)) >= cus * occ)
    if paired:
        return _lib.FA_FWD_ORDER_PAIRED
    if BH % 8 == 0 and BH * ntiles >= 16 * cus * occ:
        return _lib.FA_FWD_ORDER_HEAD_SEQUENTIAL
    return _lib.FA_FWD_ORDER_HEAVY_FIRST


_ORDER = {"heavy": _lib.FA_FWD_ORDER_HEAVY_FIRST, "paired": _lib.FA_FWD_ORDER_PAIRED,
          "seq": _lib.FA_FWD_ORDER_HEAD_SEQUENTIAL}


@pytest.mark.parametrize("Nq,Nk,BH,d,causal,cus,occ,want", [
    (4096, 4096, 32, 128, True, 256, 2, "heavy"),     # K+V of a head 2 MB: fits the L2
    (8192, 8192, 32, 128, True, 256, 2, "paired"),    # 4 MB: exactly the L2
    (8191, 8191, 32, 128, True, 256, 2, "heavy"),     # one key short of it
    (8192, 8192, 32, 128, False, 256, 2, "heavy"),    # no mask: tiles cost the same
    (16384, 16384, 32, 64, True, 256, 3, "paired"),
    (8192, 8192, 32, 64, True, 256, 3, "heavy"),
    (16384, 16384, 4, 128, True, 256, 2, "heavy"),    # 256 pairs for 512 slots
    (16384, 16384, 8, 128, True, 256, 2, "paired"),   # 512 pairs fill 512 slots
    (16300, 16300, 8, 128, True, 256, 2, "paired"),   # odd tile count (128 tiles -> 64 pairs)
    (128, 1 << 20, 4096, 128, True, 256, 2, "heavy"), # a single tile
    (256, 8192, 512, 128, True, 256, 2, "paired"),    # Nq < Nk
    (4096, 4096, 16, 256, True, 256, 1, "paired"),    # d = 256: 4 MB at N = 4096
    (2048, 2048, 512, 128, True, 256, 2, "seq"),      # 8192 workgroups: 16 rounds of 512
    (2048, 2048, 504, 128, True, 256, 2, "heavy"),    # 8064: under 16 rounds
    (2048, 2048, 516, 128, True, 256, 2, "heavy"),    # B*H not a multiple of 8
    (4096, 4096, 256, 128, False, 256, 2, "seq"),     # no mask
    (1024, 1024, 1024, 64, True, 256, 3, "heavy"),    # 8192 for 768 slots: 10.7 rounds
    (1024, 1024, 2048, 64, True, 256, 3, "seq"),
    (8192, 8192, 512, 128, True, 256, 2, "paired"),   # pairs first
    (128, 1 << 16, 8192, 128, True, 256, 2, "seq"),   # single tiles, many heads
])
def test_tile_order_rule(Nq, Nk, BH, d, causal, cus, occ, want):
    got = _lib.tile_order(Nq, BH, d, causal, Nk=Nk, cus=cus, occ=occ)
    assert got == expected_order(Nq, Nk, BH, d, causal, cus, occ)
    assert got == _ORDER[want]
    # Strict causal orders like causal; fp16 like bf16.
    assert _lib.tile_order(Nq, BH, d, "strict" if causal else False, Nk=Nk, cus=cus, occ=occ) == got
    import torch
    assert _lib.tile_order(Nq, BH, d, causal, Nk=Nk, dtype=torch.float16, cus=cus, occ=occ) == got


def test_tile_order_sweep_matches_rule():
    for Nq in (128, 256, 1000, 4096, 8192, 12345, 16384):
        for Nk in (Nq, 2 * Nq, 70000):
            for BH in (1, 8, 20, 64, 256, 1000, 1024):
                for d in (32, 64, 128, 256):
                    for occ in (1, 2, 3):
                        for causal in (True, False):
                            got = _lib.tile_order(Nq, BH, d, causal, Nk=Nk, cus=256, occ=occ)
                            assert got == expected_order(Nq, Nk, BH, d, causal, 256, occ), \
                                (Nq, Nk, BH, d, occ, causal)


def test_tile_order_argument_errors():
    lib = _lib.load()
    INV, UNS = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    bf16, f32 = _lib.FA_DTYPE_BF16, _lib.FA_DTYPE_F32
    assert lib.fa_fwd_tile_order(0, 128, 1, 128, bf16, 1, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 0, 1, 128, bf16, 1, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 0, 128, bf16, 1, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 0, bf16, 1, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 128, 7, 1, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 128, bf16, 5, 256, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 128, bf16, 1, -1, 2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 128, bf16, 1, 256, -2) == INV
    assert lib.fa_fwd_tile_order(128, 128, 1, 128, f32, 1, 256, 2) == UNS


# ---- backward work order (fa_bwd_tile_order; host only with explicit cus, occ) ----

def expected_bwd_order(B, H, Hkv, Nq, Nk, cus, occ):
    """The header's rule, per gradient kernel: head-sequential when its head
    count is a multiple of 8 and its grid is at least 16 rounds of slots."""
    dq = (B * H) % 8 == 0 and B * H * -(-Nq // BM) >= 16 * cus * occ
    dkdv = (B * Hkv) % 8 == 0 and B * Hkv * -(-Nk // BM) >= 16 * cus * occ
    return (_lib.FA_BWD_DQ_HEAD_SEQUENTIAL if dq else 0) | (_lib.FA_BWD_DKDV_HEAD_SEQUENTIAL if dkdv else 0)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,occ,want", [
    (2, 16, 16, 4096, 4096, 128, 2, 0),      # the metric backward: 2 rounds
    (4, 16, 16, 8192, 8192, 128, 2, 0),      # 8 rounds
    (8, 32, 32, 4096, 4096, 128, 2, 3),      # 16 rounds
    (8, 32, 8, 8192, 8192, 128, 2, 1),       # grouped: dK/dV's grid is 4x smaller
    (3, 20, 20, 16384, 16384, 128, 2, 0),    # 60 heads: not a multiple of 8
    (8, 32, 16, 4096, 4096, 256, 1, 3),
    (16, 32, 32, 1024, 65536, 128, 2, 2),    # Nq < Nk: only dK/dV's grid is large
])
def test_bwd_tile_order_rule(B, H, Hkv, Nq, Nk, d, occ, want):
    got = _lib.bwd_tile_order(B, H, Nq, d, Hkv=Hkv, Nk=Nk, cus=256, occ=occ)
    assert got == want == expected_bwd_order(B, H, Hkv, Nq, Nk, 256, occ)


def test_bwd_tile_order_sweep_and_errors():
    for B in (1, 2, 8, 16):
        for H, Hkv in ((16, 16), (32, 8), (12, 4)):
            for N in (128, 1000, 4096, 16384):
                for occ in (1, 2):
                    assert _lib.bwd_tile_order(B, H, N, 128, Hkv=Hkv, cus=256, occ=occ) == \
                        expected_bwd_order(B, H, Hkv, N, N, 256, occ)
    lib = _lib.load()
    INV, UNS = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_tile_order(0, 1, 1, 128, 128, 128, 256, 2) == INV
    assert lib.fa_bwd_tile_order(1, 3, 2, 128, 128, 128, 256, 2) == INV   # H % Hkv != 0
    assert lib.fa_bwd_tile_order(1, 1, 1, 128, 128, 128, -1, 2) == INV
    assert lib.fa_bwd_tile_order(1, 1, 1, 128, 128, 48, 256, 2) == UNS   # head dimension
