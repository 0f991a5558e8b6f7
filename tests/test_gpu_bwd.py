"""GPU parity of fa_bwd against the fp64 oracle's gradients (through the C-ABI)."""
import numpy as np
import pytest
import torch

import exact_io_aware_17_amd as fa
from exact_io_aware_17_amd import workloads as W

from _parity import BF16_GRAD, oracle_bwd, say, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check_grads(w: W.Workload, kv_lens=None, rel: float = 0.0):
    """max-abs <= 5e-2 (+ rel * |ref| where a gradient is too large for bf16 to
    hold within 5e-2: its half-ulp alone exceeds that above 12.8)."""
    x = W.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    kv = kv_lens
    kvd = None if kv is None else kv.to(DEV)
    say(f"bwd case B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} "
        f"kv_lens={None if kv is None else kv.tolist()}")
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_lens=kvd)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, kv_lens=kvd)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_bwd(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal, kv)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gh = to64(g)
        assert np.all(np.isfinite(gh)), name
        err = np.abs(gh - r)
        say(f"   {name} max-abs {err.max():.3e} mean-abs {err.mean():.3e} (|ref| max {np.abs(r).max():.3g})")
        assert np.all(err <= BF16_GRAD + rel * np.abs(r)), f"{name} max-abs {err.max():.3g}"
    return dq, dk, dv


def test_workload5_backward_full():
    _check_grads(W.BY_ID[5])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True, "strict"])
@pytest.mark.parametrize("N", [1, 100, 257])
def test_backward_ragged(d, causal, N):
    w = W.Workload(95, "bwd ragged", 2, 2, N, d, "bf16", causal, backward=True)
    _check_grads(w)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_padding(causal):
    w = W.Workload(96, "bwd padded", 4, 2, 320, 128, "bf16", causal, backward=True)
    kv = torch.tensor([0, 1, 200, 320], dtype=torch.int32)
    # kv_len = 1: key 0 collects dV = sum of all dO rows (|dV| ~ 60), where the
    # bf16 output's rounding step alone is 0.25; allow 2^-8 |ref| on top.
    dq, dk, dv = _check_grads(w, kv, rel=2.0 ** -8)
    # A batch with no visible key has zero gradients; keys past kv_len get none.
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    assert torch.all(dk[2, :, 200:] == 0) and torch.all(dv[2, :, 200:] == 0)


def test_backward_deterministic():
    w = W.Workload(97, "bwd det", 1, 4, 512, 128, "bf16", True, backward=True)
    x = W.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
