"""fa_fwd_ex_noalloc (the split-KV forward with its workspace in the
library's per-device scratch) against fa_fwd_ex with a caller-provided
workspace, through the C ABI: bitwise the same outputs on consecutive calls,
the second smaller than the first, and the oversize rejection."""
import pytest
import torch

import exact_io_aware_17_amd as fa
from exact_io_aware_17_amd import _lib

from _parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 64 << 20


def _inputs(B, H, Hkv, Nq, Nk, d, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(dtype).to(DEV)
    k = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype).to(DEV)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(dtype).to(DEV)
    return q, k, v


def _compare(B, H, Hkv, Nq, Nk, d, causal, seed, dtype=torch.bfloat16, kv_lens=None):
    say(f"noalloc vs fa_fwd_ex: B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
        f"{dtype}")
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed, dtype)
    need = fa.split_workspace_bytes(B, H, Nq, d, causal, Hkv, Nk, dtype)
    assert 0 < need <= SCRATCH, need  # the case splits, within the scratch
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    kvd = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
    o_ref, l_ref = fa.fwd(q, k, v, causal=causal, kv_lens=kvd, split=True, workspace=ws)
    o, l = fa.fwd_noalloc(q, k, v, causal=causal, kv_lens=kvd)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(l, l_ref)
    return o


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # Decode with grouped heads over a long cache, then a smaller decode:
    # the second call finds the first call's partial states in the scratch.
    _compare(8, 32, 8, 1, 32768, 128, True, 1701)
    _compare(2, 32, 8, 1, 8192, 128, True, 1702)
    # A causal prefill on a small grid (split tiles of 128 query rows), then
    # a smaller one with key padding, and fp16.
    _compare(1, 2, 2, 16384, 16384, 128, True, 1703)
    _compare(1, 2, 2, 8192, 8192, 64, True, 1704, kv_lens=[5000])
    _compare(1, 4, 2, 4096, 4096, 128, "strict", 1705, dtype=torch.float16)


def test_noalloc_without_a_split_and_fp32():
    # Shapes whose plan splits nothing need no scratch: same outputs as fa_fwd_ex.
    q, k, v = _inputs(2, 16, 16, 1024, 1024, 128, 1706)
    o_ref, l_ref = fa.fwd(q, k, v, causal=True, split=True)
    o, l = fa.fwd_noalloc(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    qf, kf, vf = (t[:, :2].float().contiguous() for t in (q, k, v))
    o_ref, l_ref = fa.fwd(qf, kf, vf, causal=True)
    o, l = fa.fwd_noalloc(qf, kf, vf, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_rejects_plans_beyond_the_scratch():
    # A few heads of many query tiles over a long key range split into many
    # partial states; find a shape whose plan needs more than the scratch.
    cands = [(1, 3, 3, 4096, 16384, 128, False), (1, 4, 4, 4096, 16384, 128, False),
             (1, 2, 2, 4096, 65536, 128, False)]
    for (B, H, Hkv, Nq, Nk, d, causal) in cands:
        need = fa.split_workspace_bytes(B, H, Nq, d, causal, Hkv, Nk)
        if need > SCRATCH:
            break
    else:
        pytest.skip("no candidate shape splits beyond the scratch on this device")
    say(f"oversize: B={B} H={H} Nq={Nq} Nk={Nk} d={d} needs {need} bytes")
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, 1707)
    with pytest.raises(_lib.FaError) as e:
        fa.fwd_noalloc(q, k, v, causal=causal)
    assert e.value.status == _lib.FA_ERR_UNSUPPORTED
    # The scratch stays usable after the rejection.
    _compare(2, 32, 8, 1, 8192, 128, True, 1702)
