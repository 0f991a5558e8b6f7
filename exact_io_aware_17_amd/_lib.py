"""ctypes binding of libfa (include/fa.h): argument marshalling only.

Every step of the attention runs in libfa's gfx950 kernels. PyTorch supplies
device memory (output and workspace tensors) and the current HIP stream.
There is no fallback: if libfa.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
FA_MASK_CAUSAL_STRICT = 2
FA_DTYPE_BF16 = 0
FA_DTYPE_F16 = 1
FA_DTYPE_F32 = 2
ABI_VERSION = 12

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

# Exported symbol -> (restype, argtypes), in the order include/fa.h declares them.
SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "fa_fwd_ex_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "fa_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                       ctypes.c_size_t, _vp]),
    "fa_fwd_ex_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                               _vp, _vp]),
    "fa_fwd_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                    _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "fa_bwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                       _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "fa_fwd_schedule": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp]),
    "fa_fwd_tile_order": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "fa_bwd_tile_order": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "fa_fwd_block_keys": (_i, [_i, _i, _i, _i, _i, _i]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_abi_version": (_i, []),
}


class FaError(RuntimeError):
    """A libfa call returned a non-zero status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once (after torch, so it binds to the HIP runtime torch uses)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"libfa.so not found at {path}; build it with `python -m exact_io_aware_17_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.fa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libfa ABI {lib.fa_abi_version()} != expected {ABI_VERSION}")
    if path == LIB_PATH:
        _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != FA_OK:
        raise FaError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def mask_kind(causal) -> int:
    """causal: False (no mask), True (key j visible to query i iff j <= i) or
    "strict" (iff j < i)."""
    if isinstance(causal, str):
        if causal != "strict":
            raise ValueError("causal must be False, True or 'strict'")
        return FA_MASK_CAUSAL_STRICT
    return FA_MASK_CAUSAL if causal else FA_MASK_NONE


_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16,
           torch.float32: FA_DTYPE_F32}


def dtype_code(dtype: torch.dtype) -> int:
    """fa_dtype of a torch dtype (bfloat16, float16 or float32)."""
    if dtype not in _DTYPES:
        raise ValueError("tensors must be bfloat16, float16 or float32")
    return _DTYPES[dtype]


def default_scale(d: int) -> float:
    """float32(1/sqrt(d)), the value every path receives."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def _check_qkv(q, k, v):
    """q [B, H, Nq, d]; k, v [B, Hkv, Nk, d] with H a multiple of Hkv.
    Returns (B, H, Hkv, Nq, Nk, d)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-d ([B, H, N, d])")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape [B, Hkv, Nk, d]")
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k, v must agree in batch and head dimension")
    if Hkv == 0 or H % Hkv != 0:
        raise ValueError("the query heads must be a multiple of the K/V heads")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    return B, H, Hkv, Nq, Nk, d


def _kv_ptr(kv_lens, B, dev):
    if kv_lens is None:
        return None
    if kv_lens.dtype != torch.int32 or kv_lens.device != dev or kv_lens.shape != (B,) \
            or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be a contiguous int32 [B] tensor on the inputs' device")
    return kv_lens.data_ptr()


# Zero-filled fa_fwd_ex workspaces, one per (device, stream), grown on demand:
# every completed call leaves the counter region zero, and calls that share a
# workspace must be ordered, which calls on one stream are. Split forwards on
# two streams of a device therefore never share one.
_FWD_WS = {}
_FWD_WS_BYTES = {}


def split_workspace_bytes(B: int, H: int, N: int, d: int, causal=False,
                          Hkv: Optional[int] = None, Nk: Optional[int] = None,
                          dtype: torch.dtype = torch.bfloat16) -> int:
    """fa_fwd_ex_workspace_bytes for the current device (memoised per shape);
    N is the query rows, Hkv and Nk default to H and N."""
    Hkv = H if Hkv is None else Hkv
    Nk = N if Nk is None else Nk
    code = dtype_code(dtype)
    key = (torch.cuda.current_device() if torch.cuda.is_available() else -1, B, H, Hkv, N, Nk,
           d, code, mask_kind(causal))
    n = _FWD_WS_BYTES.get(key)
    if n is None:
        n = int(load().fa_fwd_ex_workspace_bytes(B, H, Hkv, N, Nk, d, code, mask_kind(causal)))
        _FWD_WS_BYTES[key] = n
    return n


def _fwd_workspace(dev: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), stream)
    ws = _FWD_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            # The old buffer may still be in use by work queued on `stream`:
            # let the caching allocator reuse it only after that work.
            ws.record_stream(torch.cuda.ExternalStream(stream, device=dev))
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _FWD_WS[key] = ws
    return ws


def schedule(N: int, BH: int, causal, cus: int, occ: int, Nk: Optional[int] = None,
             d: int = 128):
    """fa_fwd_schedule: (items, nslots) of fa_fwd_ex's work plan (host only);
    N query rows, Nk keys (default N), head dimension d."""
    lib = load()
    buf = (ctypes.c_uint32 * 4096)()
    ns = ctypes.c_int(0)
    n = lib.fa_fwd_schedule(N, N if Nk is None else Nk, BH, d, mask_kind(causal), cus, occ, buf,
                            4096, ctypes.byref(ns))
    if n < 0:
        raise FaError("fa_fwd_schedule", n, status_string(n))
    return [int(buf[i]) for i in range(n)], int(ns.value)


FA_FWD_ORDER_HEAVY_FIRST = 0
FA_FWD_ORDER_PAIRED = 1
FA_FWD_ORDER_HEAD_SEQUENTIAL = 2


def tile_order(N: int, BH: int, d: int, causal, Nk: Optional[int] = None,
               dtype: torch.dtype = torch.bfloat16, cus: int = 0, occ: int = 0) -> int:
    """fa_fwd_tile_order: FA_FWD_ORDER_HEAVY_FIRST, FA_FWD_ORDER_PAIRED or
    FA_FWD_ORDER_HEAD_SEQUENTIAL for N query rows against Nk keys (default N)
    and BH query heads; cus = occ = 0 asks for the current device's compute
    units and occupancy."""
    n = int(load().fa_fwd_tile_order(N, N if Nk is None else Nk, BH, d, dtype_code(dtype),
                                     mask_kind(causal), cus, occ))
    if n < 0:
        raise FaError("fa_fwd_tile_order", n, status_string(n))
    return n


FA_BWD_DQ_HEAD_SEQUENTIAL = 1
FA_BWD_DKDV_HEAD_SEQUENTIAL = 2


def bwd_tile_order(B: int, H: int, N: int, d: int, Hkv: Optional[int] = None,
                   Nk: Optional[int] = None, cus: int = 0, occ: int = 0) -> int:
    """fa_bwd_tile_order: which gradient kernels run each XCD's heads one after
    another (FA_BWD_*_HEAD_SEQUENTIAL bits) for N query rows over Nk keys
    (default N) and Hkv K/V heads (default H)."""
    n = int(load().fa_bwd_tile_order(B, H, H if Hkv is None else Hkv, N, N if Nk is None else Nk,
                                     d, cus, occ))
    if n < 0:
        raise FaError("fa_bwd_tile_order", n, status_string(n))
    return n


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=False,
        scale: Optional[float] = None, kv_lens: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        split: bool = False, workspace: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward of q [B, H, Nq, d] over k, v [B, Hkv, Nk, d]. Returns (O, lse).

    bfloat16 with Hkv = H, Nq = Nk and split False calls fa_fwd; float32 with
    Hkv = H and Nq = Nk calls fa_fwd_f32; every other case (float16, grouped
    K/V heads, Nq != Nk, split) calls fa_fwd_ex. With split=True (16-bit
    types) fa_fwd_ex may split the key range of heavy query tiles over several
    workgroups, using `workspace` (a uint8 device tensor whose first 64 KiB
    are zero, of at least split_workspace_bytes(...) bytes) or, if None, a
    per-device cached one.
    """
    B, H, Hkv, Nq, Nk, d = _check_qkv(q, k, v)
    plain = (Hkv == H and Nq == Nk)
    code = dtype_code(q.dtype)
    if scale is None:
        scale = default_scale(d)
    if split and code == FA_DTYPE_F32:
        raise ValueError("split-KV is a 16-bit path")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must match q")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    kvp = _kv_ptr(kv_lens, B, q.device)
    lib = load()
    mask = mask_kind(causal)
    tensors = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse))
    with torch.cuda.device(q.device):
        stream = _stream(q.device)
        if code == FA_DTYPE_F32 and plain:
            fn_name = "fa_fwd_f32"
            st = lib.fa_fwd_f32(*tensors, B, H, Nq, d, float(scale), mask, kvp, stream)
        elif code == FA_DTYPE_BF16 and plain and not split:
            fn_name = "fa_fwd"
            st = lib.fa_fwd(*tensors, B, H, Nq, d, float(scale), mask, kvp, stream)
        else:
            fn_name = "fa_fwd_ex"
            ws_ptr, ws_bytes = None, 0
            if split and workspace is None:
                need = split_workspace_bytes(B, H, Nq, d, causal, Hkv, Nk, q.dtype)
                if need > 0:
                    workspace = _fwd_workspace(q.device, stream, need)
            if split and workspace is not None:
                if workspace.device != q.device or not workspace.is_contiguous():
                    raise ValueError("workspace must be a contiguous tensor on q's device")
                ws_ptr = workspace.data_ptr()
                ws_bytes = workspace.numel() * workspace.element_size()
            st = lib.fa_fwd_ex(*tensors, B, H, Hkv, Nq, Nk, d, code, float(scale), mask, kvp,
                               ws_ptr, ws_bytes, stream)
    _check(fn_name, st)
    return out, lse


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=False,
                scale: Optional[float] = None, kv_lens: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fa_fwd_ex_noalloc: the split-KV forward of fwd(split=True) with its
    workspace in the library's per-device scratch (no device allocation by
    the library; `out` and `lse`, if given, make the call allocation-free
    here too). Calls on one device must be ordered (they share the scratch)."""
    B, H, Hkv, Nq, Nk, d = _check_qkv(q, k, v)
    code = dtype_code(q.dtype)
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must match q")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    kvp = _kv_ptr(kv_lens, B, q.device)
    lib = load()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv,
                                   Nq, Nk, d, code, float(scale), mask_kind(causal), kvp,
                                   _stream(q.device))
    _check("fa_fwd_ex_noalloc", st)
    return out, lse


def block_keys(B: int, H: int, N: int, d: int, causal=False, Nk: Optional[int] = None) -> int:
    """fa_fwd_block_keys: keys per streamed block of the forward launch on the
    current device."""
    n = int(load().fa_fwd_block_keys(B, H, N, N if Nk is None else Nk, d, mask_kind(causal)))
    if n < 0:
        raise FaError("fa_fwd_block_keys", n, status_string(n))
    return n


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    """fa_bwd_workspace_bytes; N is the query rows."""
    return int(load().fa_bwd_workspace_bytes(B, H, N, d))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
        lse: torch.Tensor, dout: torch.Tensor, causal=False,
        scale: Optional[float] = None, kv_lens: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward (bfloat16 or float16): fa_bwd for bfloat16 with Hkv = H and
    Nq = Nk, else fa_bwd_ex. Returns (dQ [B, H, Nq, d], dK, dV [B, Hkv, Nk, d])."""
    B, H, Hkv, Nq, Nk, d = _check_qkv(q, k, v)
    code = dtype_code(q.dtype)
    if code == FA_DTYPE_F32:
        raise ValueError("the backward takes bfloat16 or float16 tensors")
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must match q")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    if scale is None:
        scale = default_scale(d)
    lib = load()
    wsb = int(lib.fa_bwd_workspace_bytes(B, H, Nq, d))
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < wsb or workspace.device != q.device \
            or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous device tensor of {wsb} bytes")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    kvp = _kv_ptr(kv_lens, B, q.device)
    tensors = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
               _ptr(dv), _ptr(workspace))
    with torch.cuda.device(q.device):
        stream = _stream(q.device)
        if code == FA_DTYPE_BF16 and Hkv == H and Nq == Nk:
            fn_name = "fa_bwd"
            st = lib.fa_bwd(*tensors, B, H, Nq, d, float(scale), mask_kind(causal), kvp, stream)
        else:
            fn_name = "fa_bwd_ex"
            st = lib.fa_bwd_ex(*tensors, B, H, Hkv, Nq, Nk, d, code, float(scale),
                               mask_kind(causal), kvp, stream)
    _check(fn_name, st)
    return dq, dk, dv
