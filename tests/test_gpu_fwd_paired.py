"""GPU parity of the paired causal tile order against the fp64 oracle.

Under the causal mask, when one head's K and V outgrow one XCD's L2 (4 MB),
the forward gives each workgroup two query tiles: tile ntiles-1-r with its
keys in ascending order, then tile r with its keys in descending order
(fa_fwd_tile_order, FA_FWD_ORDER_PAIRED). The online recurrence and the block
merge are exact for any block order ("The Flash Attention"; "Exercises", a
common reference gives the same result), so the outputs must match the
definition to the same tolerances as the heavy-first order. Each case first
checks that the device really takes the paired order for it, then compares
whole heads (every row) and sampled rows of every head with the oracle: the
rows at both ends of every query tile, the middle of the sequence, and the
ragged tail. The cases cover an even and an odd number of tiles, a ragged
last tile, B*H not a multiple of 8 (heads dealt without the per-XCD
grouping), grouped K/V heads, Nq < Nk, key padding with the strict mask,
fp16, and d = 64 and 256.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa
from exact_io_aware_17_amd import workloads as W

from _parity import (BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, F16_O_MAX,
                     F16_O_MEAN, check_lse, check_o, oracle_fwd, say, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BM = 128

# (B, H, Hkv, Nq, Nk, d, dtype, causal, kv_lens, whole heads)
CASES = [
    (1, 32, 32, 8192, 8192, 128, "bf16", True, None, [(0, 0), (0, 21)]),
    (1, 24, 24, 8300, 8300, 128, "bf16", True, None, [(0, 0), (0, 13)]),  # 65 tiles, ragged
    (1, 20, 20, 8192, 8192, 128, "bf16", True, None, [(0, 7)]),           # B*H % 8 != 0
    (2, 16, 16, 8192, 8192, 128, "bf16", "strict", [8192, 3001], [(0, 3), (1, 9)]),
    (1, 32, 8, 8192, 8192, 128, "bf16", True, None, [(0, 5)]),            # 4 heads per K/V head
    (4, 32, 32, 1024, 8192, 128, "bf16", True, None, [(3, 31)]),          # continuation
    (1, 32, 32, 8192, 8192, 128, "f16", True, None, [(0, 30)]),
    (1, 32, 32, 16384, 16384, 64, "bf16", True, None, [(0, 2)]),
    (1, 16, 16, 4096, 4096, 256, "bf16", True, None, [(0, 0), (0, 15)]),
]


def _ids(c):
    B, H, Hkv, Nq, Nk, d, dt, causal, kv, _ = c
    tag = {True: "c", "strict": "s"}[causal]
    return f"B{B}H{H}g{Hkv}q{Nq}k{Nk}d{d}{dt}{tag}{'' if kv is None else 'kv'}"


def _sample_rows(Nq):
    rows = set()
    for t in range(0, Nq, BM):
        rows.update((t, min(Nq, t + BM) - 1))
    rows.update((Nq // 2 - 1, Nq // 2, Nq - 1))
    return sorted(r for r in rows if 0 <= r < Nq)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_paired_order_matches_oracle(case):
    B, H, Hkv, Nq, Nk, d, dt, causal, kvl, whole = case
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    order = fa.tile_order(Nq, B * H, d, causal, Nk=Nk, dtype=dtype)
    say(f"case {_ids(case)}: tile order {order}")
    assert order == fa.FA_FWD_ORDER_PAIRED
    g = torch.Generator().manual_seed(Nq * 31 + H * 7 + d)
    q = torch.randn(B, H, Nq, d, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    scale = W.Workload(0, "", B, H, Nq, d, dt, causal).scale
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                    kv_lens=None if kv is None else kv.to(DEV))
    torch.cuda.synchronize()
    o_g, lse_g = to64(o), to64(lse)
    assert np.all(np.isfinite(o_g))
    o_max, o_mean = (BF16_O_MAX, BF16_O_MEAN) if dt == "bf16" else (F16_O_MAX, F16_O_MEAN)
    # Sampled rows of every head.
    rows = _sample_rows(Nq)
    say(f"   {len(rows)} sampled rows of all {B * H} heads")
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv, rows=rows)
    check_o(o_g[:, :, rows], o_ref, o_max)
    check_lse(lse_g[:, :, rows], lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    # Whole heads, in row chunks.
    for b, h in whole:
        say(f"   batch {b} head {h}: all {Nq} rows")
        chunk = 4096
        o_ref = np.empty_like(o_g[b, h])
        lse_ref = np.empty_like(lse_g[b, h])
        hk = h // (H // Hkv)
        qh, kh, vh = q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1]
        kvb = None if kv is None else kv[b:b + 1]
        for r0 in range(0, Nq, chunk):
            rr = list(range(r0, min(Nq, r0 + chunk)))
            orf, lrf = oracle_fwd(qh, kh, vh, scale, causal, kvb, rows=rr)
            o_ref[r0:r0 + len(rr)] = orf[0, 0]
            lse_ref[r0:r0 + len(rr)] = lrf[0, 0]
        check_o(o_g[b, h], o_ref, o_max, o_mean)
        check_lse(lse_g[b, h], lse_ref, BF16_LSE_ABS, BF16_LSE_REL)


def test_workload4_takes_the_paired_order():
    """The padded N = 16384 workload (checked whole-head against the oracle in
    test_gpu_fwd) runs the paired order."""
    w = W.BY_ID[4]
    assert fa.tile_order(w.N, w.B * w.H, w.d, w.causal) == fa.FA_FWD_ORDER_PAIRED


def test_metric_shape_keeps_the_heavy_first_order():
    w = W.BY_ID[5]
    assert fa.tile_order(w.N, w.B * w.H, w.d, w.causal) == fa.FA_FWD_ORDER_HEAVY_FIRST
