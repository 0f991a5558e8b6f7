"""libfa_probe (the matrix-core and HBM -> LDS rate probes the benchmark
measures beside the forward and the decode) loads, exports what
include/fa_probe.h declares, rejects bad arguments before any HIP call, and
states its FLOPs and bytes per launch."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_io_aware_17_amd", "libfa_probe.so")


def _load():
    assert os.path.exists(LIB), "libfa_probe.so is not built (python -m exact_io_aware_17_amd.build)"
    lib = ctypes.CDLL(LIB)
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.fa_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.fa_probe_stream_lds.restype = ctypes.c_int
    lib.fa_probe_stream_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.fa_probe_stream_lds_bytes.restype = ctypes.c_double
    lib.fa_probe_stream_lds_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def test_exports_what_the_header_declares():
    with open(os.path.join(ROOT, "include", "fa_probe.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_probe_\w+)\s*\(", text)))
    assert names == ["fa_probe_mfma_bf16", "fa_probe_mfma_bf16_flops", "fa_probe_stream_lds",
                     "fa_probe_stream_lds_bytes"]
    lib = _load()
    for n in names:
        assert hasattr(lib, n), n


def test_bad_arguments_are_rejected_before_launch():
    lib = _load()
    sink = ctypes.c_void_p(0x10000000)  # never dereferenced: every call fails validation
    assert lib.fa_probe_mfma_bf16(0, 10, sink, None) == -1
    assert lib.fa_probe_mfma_bf16(-4, 10, sink, None) == -1
    assert lib.fa_probe_mfma_bf16(512, 0, sink, None) == -1
    assert lib.fa_probe_mfma_bf16(512, 10, None, None) == -1
    src = ctypes.c_void_p(0x20000000)
    assert lib.fa_probe_stream_lds(None, 512, 8, sink, None) == -1
    assert lib.fa_probe_stream_lds(src, 512, 8, None, None) == -1
    assert lib.fa_probe_stream_lds(src, 0, 8, sink, None) == -1
    assert lib.fa_probe_stream_lds(src, 512, 0, sink, None) == -1
    assert lib.fa_probe_stream_lds(src, (1 << 20) + 1, 8, sink, None) == -1
    assert lib.fa_probe_stream_lds(src, 512, (1 << 16) + 1, sink, None) == -1


def test_flops_per_launch():
    lib = _load()
    # 4 waves per workgroup, 4 MFMAs per round, 32 x 32 x 16 x 2 FLOPs each
    assert lib.fa_probe_mfma_bf16_flops(512, 512) == 512 * 4 * 512 * 4 * 32 * 32 * 16 * 2
    assert lib.fa_probe_mfma_bf16_flops(0, 5) == 0.0


def test_stream_bytes_per_launch():
    lib = _load()
    assert lib.fa_probe_stream_lds_bytes(512, 64) == 512 * 64 * 32768
    assert lib.fa_probe_stream_lds_bytes(512, 0) == 0.0
