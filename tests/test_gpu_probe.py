"""The HBM -> LDS streaming probe that the decode figures are compared with
reads every block it is given: with a source of bf16 ones each workgroup's
sum is 32 per 32 KB block (wave 0 adds one element per lane group of 16
bytes, 32 per block), for even and odd block counts."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_io_aware_17_amd", "libfa_probe.so")


@pytest.mark.parametrize("workgroups,blocks", [(512, 8), (300, 5), (1, 1)])
def test_stream_probe_reads_every_block(workgroups, blocks):
    lib = ctypes.CDLL(LIB)
    lib.fa_probe_stream_lds.restype = ctypes.c_int
    lib.fa_probe_stream_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    print(f"case stream probe workgroups={workgroups} blocks={blocks}", flush=True)
    src = torch.ones(workgroups * blocks * 32768 // 2, dtype=torch.bfloat16, device=dev)
    sums = torch.full((workgroups,), -1.0, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev)
    assert lib.fa_probe_stream_lds(ctypes.c_void_p(src.data_ptr()), workgroups, blocks,
                                   ctypes.c_void_p(sums.data_ptr()),
                                   ctypes.c_void_p(st.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(sums.cpu(), torch.full((workgroups,), 32.0 * blocks))
