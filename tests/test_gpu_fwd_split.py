"""GPU parity of split-KV (fa_fwd_ex with a workspace): the heaviest query tiles cut into key
ranges whose partial states are merged by the last part to arrive.

Both paths (fa_fwd_ex with the workspace, and fa_fwd with one workgroup per tile) are
compared with the fp64 oracle on the same inputs; the split path must be
bitwise reproducible and must leave its arrival counters at zero. The shapes
have few heads, so that the plan splits them.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa

from _parity import BF16_LSE_ABS, BF16_LSE_REL, BF16_O_MAX, BF16_O_MEAN, check_lse, check_o, \
    oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, N, d, causal, kv_lens)
CASES = [
    (1, 1, 1024, 128, False, None),       # every tile in 4 parts
    (1, 2, 1536, 64, True, [1400]),       # 64-key blocks (d = 64)
    (2, 3, 1000, 128, True, None),        # ragged last tile
    (2, 2, 1024, 64, False, [0, 333]),    # an empty batch and parts beyond kv_len
    (1, 2, 4096, 128, True, None),
    (2, 1, 2048, 128, True, [2048, 700]),
    (1, 2, 2048, 128, "strict", None),    # row 0 of every head sees no key
]


def _inputs(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16) for _ in range(3))
    return q, k, v


def _ids(c):
    B, H, N, d, causal, kv = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"B{B}H{H}N{N}d{d}{tag}{'' if kv is None else 'kv'}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_split_and_unsplit_match_oracle(case):
    B, H, N, d, causal, kvl = case
    say(f"case split B={B} H={H} N={N} d={d} causal={causal} kv_lens={kvl}")
    need = fa.split_workspace_bytes(B, H, N, d, causal)
    assert need > 0, "the plan was expected to split this shape"
    q, k, v = _inputs(B, H, N, d, 1700 + N + d)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    kvd = None if kv is None else kv.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    scale = fa.default_scale(d)
    o_s, lse_s = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd, split=True,
                        workspace=ws)
    o_u, lse_u = fa.fwd(qd, kd, vd, causal=causal, scale=scale, kv_lens=kvd)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    for o, lse in ((o_s, lse_s), (o_u, lse_u)):
        check_o(to64(o), o_ref, BF16_O_MAX, BF16_O_MEAN)
        check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    # The arrival counters (first 64 KiB of the workspace) are back at zero.
    assert int(ws[:65536].view(torch.int32).abs().sum().item()) == 0


def test_split_is_bitwise_reproducible_and_reusable():
    B, H, N, d = 1, 4, 4096, 128
    say(f"case split-repeat B={B} H={H} N={N} d={d}")
    need = fa.split_workspace_bytes(B, H, N, d, True)
    assert need > 0
    q, k, v = (t.to(DEV) for t in _inputs(B, H, N, d, 1717))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    outs = [fa.fwd(q, k, v, causal=True, split=True, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0])
        assert torch.equal(lse, outs[0][1])
    # A smaller shape on the same (larger) workspace right after, whose
    # counters would overlap the first shape's partial states if they were
    # laid out per shape.
    q2, k2, v2 = (t[:1, :2, :1000].contiguous() for t in (q, k, v))
    assert 0 < fa.split_workspace_bytes(1, 2, 1000, d, True) <= need
    o2, lse2 = fa.fwd(q2, k2, v2, causal=True, split=True, workspace=ws)
    o2u, lse2u = fa.fwd(q2, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o2.float() - o2u.float())).item() <= 2 * BF16_O_MAX
    assert torch.max(torch.abs(lse2 - lse2u)).item() <= 2e-3


def test_short_workspace_runs_unsplit():
    B, H, N, d = 1, 2, 1024, 128
    need = fa.split_workspace_bytes(B, H, N, d, True)
    assert need > 0
    q, k, v = (t.to(DEV) for t in _inputs(B, H, N, d, 1718))
    short = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    o_a, lse_a = fa.fwd(q, k, v, causal=True, split=True, workspace=short)
    o_b, lse_b = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(lse_a, lse_b)
    assert int(short.abs().sum().item()) == 0  # untouched


def test_metric_shape_is_not_split():
    # Several waves of workgroups: the plan keeps one workgroup per tile.
    assert fa.split_workspace_bytes(2, 16, 4096, 128, True) == 0


# Decode over long caches: one query per head, grouped K/V heads packed as the
# rows of a single query tile, whose key range is cut into more than 16 parts
# (up to 64); the last part to arrive merges with all four waves, each taking
# a share of the d columns of the one wave that holds rows.
# (B, H, Hkv, Nk, d, dtype, causal, kv_lens)
DECODE = [
    (1, 32, 8, 131072, 128, torch.bfloat16, True, None),
    (1, 8, 8, 32768, 64, torch.bfloat16, True, None),         # d = 64: two waves merge
    (1, 16, 4, 32768, 256, torch.bfloat16, True, None),       # d = 256: two d tiles per wave
    (1, 8, 2, 32768, 32, torch.bfloat16, False, None),        # d = 32: one wave merges
    (1, 12, 4, 40000, 96, torch.float16, True, None),         # d = 96, fp16, ragged last block
    (2, 8, 2, 65536, 128, torch.bfloat16, True, [65536, 0]),  # an empty sequence
    (1, 4, 4, 50000, 128, torch.bfloat16, "strict", [30001]),  # unpacked: one row per head
]


def _decode_ids(c):
    B, H, Hkv, Nk, d, dt, causal, kv = c
    tag = {False: "", True: "c", "strict": "s"}[causal]
    return f"B{B}H{H}g{Hkv}k{Nk}d{d}{'f16' if dt == torch.float16 else ''}{tag}{'' if kv is None else 'kv'}"


@pytest.mark.parametrize("case", DECODE, ids=[_decode_ids(c) for c in DECODE])
def test_decode_with_many_parts_matches_oracle(case):
    B, H, Hkv, Nk, d, dtype, causal, kvl = case
    say(f"case decode B={B} H={H} Hkv={Hkv} Nk={Nk} d={d} {dtype} causal={causal} kv_lens={kvl}")
    g = torch.Generator().manual_seed(1900 + Nk + d)
    q = torch.randn(B, H, 1, d, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype)
    kv = None if kvl is None else torch.tensor(kvl, dtype=torch.int32)
    need = fa.split_workspace_bytes(B, H, 1, d, causal, Hkv, Nk, dtype)
    assert need > 0, "the plan was expected to split this shape"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                    kv_lens=None if kv is None else kv.to(DEV), split=True, workspace=ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, causal, kv)
    tol = (BF16_O_MAX, BF16_O_MEAN) if dtype == torch.bfloat16 else (5e-3, 5e-4)
    check_o(to64(o), o_ref, *tol)
    check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    assert int(ws[:65536].view(torch.int32).abs().sum().item()) == 0
    if kvl is not None and 0 in kvl:
        b0 = kvl.index(0)
        assert torch.all(o[b0] == 0).item() and torch.all(torch.isneginf(lse[b0])).item()


def test_decode_plans_use_more_than_sixteen_parts():
    """The decode shapes above take plans of more than 16 parts at any
    occupancy from 1 to 4 workgroups per compute unit, so that the many-part
    merge is what their parity cases check. Launch shape: B * Hkv heads of
    H / Hkv rows when grouped heads are packed; the strict mask and H = Hkv
    keep one row per head."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, H, Hkv, Nk, d, _, causal, _ in DECODE:
        packed = H != Hkv and causal != "strict"
        rows, heads = (H // Hkv, B * Hkv) if packed else (1, B * H)
        for occ in (1, 2, 3, 4):
            items, nslots = fa.schedule(rows, heads, causal, cus, occ, Nk=Nk, d=d)
            assert len(items) > 16 and nslots == len(items), (B, H, Hkv, Nk, d, occ, len(items))


@pytest.mark.parametrize("Nq", [40, 100])
def test_short_query_chunk_with_many_parts(Nq):
    """A chunk of Nq < 128 queries after a long cache: one query tile per head
    split into more than 16 parts, with rows in two (Nq = 40) or four waves
    (Nq = 100), so the last part merges each wave's own rows."""
    B, H, Nk, d = 1, 4, 40000, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for occ in (1, 2, 3, 4):
        assert len(fa.schedule(Nq, B * H, True, cus, occ, Nk=Nk, d=d)[0]) > 16
    say(f"case chunk B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    g = torch.Generator().manual_seed(1950 + Nq)
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    need = fa.split_workspace_bytes(B, H, Nq, d, True, H, Nk)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale, split=True,
                    workspace=ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, scale, True)
    check_o(to64(o), o_ref, BF16_O_MAX, BF16_O_MEAN)
    check_lse(to64(lse), lse_ref, BF16_LSE_ABS, BF16_LSE_REL)
    assert int(ws[:65536].view(torch.int32).abs().sum().item()) == 0
