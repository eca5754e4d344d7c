"""Thin ctypes binding of libfa.so (declared in include/fa.h).

Argument marshalling only: tensors are checked, outputs allocated with torch
(device memory is torch's), and the C entry points are called on the current
torch stream.  Every step of the attention computation runs in the library's
HIP kernels.  If libfa.so is missing this module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

from .build_lib import LIB_PATH

FA_OK = 0
FA_FP16 = 0
FA_BF16 = 1

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class FaError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__("%s%s" % (what + ": " if what else "", status_str(status)))


class FaOptions(ctypes.Structure):
    """struct fa_options of include/fa.h (the optional features of a call)."""
    _fields_ = [("h_kv", ctypes.c_int64), ("mask_tiles", ctypes.c_void_p), ("dropout", ctypes.c_int),
                ("dropout_p", ctypes.c_float), ("dropout_seed", ctypes.c_uint64),
                ("dropout_offset", ctypes.c_uint64), ("num_splits", ctypes.c_int)]


def options(h_kv=0, tiles=0, dropout=None, num_splits=0):
    """FaOptions from plain values: tiles is a device address (0: no mask),
    dropout is None or (p, seed, offset)."""
    o = FaOptions()
    o.h_kv = int(h_kv)
    o.mask_tiles = int(tiles) or None
    if dropout is not None:
        p, seed, offset = dropout
        o.dropout, o.dropout_p, o.dropout_seed, o.dropout_offset = 1, float(p), int(seed), int(offset)
    o.num_splits = int(num_splits)
    return o


_lib = None


def library_path():
    return os.environ.get("FA_LIBRARY", LIB_PATH)


def load_library():
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError("libfa.so is not built (%s); run __graft_entry__.build() or "
                          "python -m exact_attention_25_amd.build_lib" % path)
    lib = ctypes.CDLL(path)
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                           ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                           ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_fwd_splitkv_num_splits.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.fa_fwd_splitkv_num_splits.restype = ctypes.c_int
    lib.fa_fwd_kernel_name.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.fa_fwd_kernel_name.restype = ctypes.c_char_p
    lib.fa_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_mask_tiles_bytes.argtypes = [_i64, _i64]
    lib.fa_mask_tiles_bytes.restype = ctypes.c_size_t
    lib.fa_mask_tiles.argtypes = [_vp, _i64, _i64, _vp, ctypes.c_size_t, _vp]
    lib.fa_mask_tiles.restype = ctypes.c_int
    _opt = ctypes.POINTER(FaOptions)
    lib.fa_fwd_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                              ctypes.c_int, _opt, _vp, ctypes.c_size_t, _vp]
    lib.fa_fwd_ex.restype = ctypes.c_int
    lib.fa_bwd_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int,
                              ctypes.c_float, ctypes.c_int, _opt, _vp, ctypes.c_size_t, _vp]
    lib.fa_bwd_ex.restype = ctypes.c_int
    lib.fa_fwd_ex_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _opt]
    lib.fa_fwd_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_ex_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _opt]
    lib.fa_bwd_ex_workspace_bytes.restype = ctypes.c_size_t
    _u64 = ctypes.c_uint64
    lib.fa_dropout_mask.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_float, _u64, _u64, _vp]
    lib.fa_dropout_mask.restype = ctypes.c_int
    lib.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                   ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp]
    lib.fa_bwd_noalloc.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status):
    return load_library().fa_status_str(int(status)).decode()


# ---- raw entry points: plain integers as pointers, same names as the C ABI ----
def fa_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, stream):
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, D, int(causal), float(scale), int(dtype), stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype,
           workspace, workspace_bytes, stream):
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, int(causal),
                                 float(scale), int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype, stream):
    return load_library().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, int(causal),
                                         float(scale), int(dtype), stream)


def fa_fwd_ex(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, opt, workspace, workspace_bytes, stream):
    """fa_fwd_ex; opt is an FaOptions or None."""
    return load_library().fa_fwd_ex(q, k, v, o, lse, B, H, N, D, int(causal), float(scale), int(dtype),
                                    ctypes.byref(opt) if opt is not None else None, workspace, workspace_bytes,
                                    stream)


def fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype, opt, workspace,
              workspace_bytes, stream):
    """fa_bwd_ex; opt is an FaOptions or None."""
    return load_library().fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, int(causal), float(scale),
                                    int(dtype), ctypes.byref(opt) if opt is not None else None, workspace,
                                    workspace_bytes, stream)


def fwd_ex_workspace_bytes(B, H, N, D, causal, dtype, opt=None):
    return int(load_library().fa_fwd_ex_workspace_bytes(B, H, N, D, int(causal), int(dtype),
                                                        ctypes.byref(opt) if opt is not None else None))


def bwd_ex_workspace_bytes(B, H, N, D, causal, dtype, opt=None):
    return int(load_library().fa_bwd_ex_workspace_bytes(B, H, N, D, int(causal), int(dtype),
                                                        ctypes.byref(opt) if opt is not None else None))


def splitkv_num_splits(B, H, N, D, causal):
    """fa_fwd_splitkv_num_splits: the library's split count for a shape."""
    return int(load_library().fa_fwd_splitkv_num_splits(B, H, N, D, int(causal)))


def fwd_kernel_name(B, H, N, D, causal):
    """fa_fwd_kernel_name: the forward kernel fa_fwd runs for this shape."""
    return load_library().fa_fwd_kernel_name(B, H, N, D, int(causal)).decode()


def bwd_workspace_bytes(B, H, N, D, causal, dtype):
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, D, int(causal), int(dtype)))


def fa_dropout_mask(keep, B, H, N, dropout_p, seed, offset, stream):
    return load_library().fa_dropout_mask(keep, B, H, N, float(dropout_p), int(seed), int(offset), stream)


def fa_mask_tiles_bytes(B, N):
    return int(load_library().fa_mask_tiles_bytes(B, N))


def fa_mask_tiles(key_mask, B, N, tiles, tiles_bytes, stream):
    return load_library().fa_mask_tiles(key_mask, B, N, tiles, tiles_bytes, stream)


# ---- torch-tensor convenience wrappers ----
def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError("attention tensors must be float16 or bfloat16, got %s" % t.dtype)


def _check(tensors, shape, dtype, device):
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if t.dtype != dtype:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous [B, H, N, D]" % name)


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _kv_heads(q, k):
    """H_kv from k's shape [B, H_kv, N, D] (grouped heads when H_kv < H)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, D] and [B, H_kv, N, D]")
    B, H, N, D = q.shape
    hkv = k.shape[1]
    if hkv < 1 or H % hkv != 0:
        raise ValueError("k has %d heads, which does not divide the %d query heads" % (hkv, H))
    return hkv


def _fwd(q, k, v, causal, scale, out, lse, opt, workspace, what):
    """Checks, allocations and one fa_fwd / fa_fwd_ex call; opt None = plain."""
    import torch
    hkv = _kv_heads(q, k)
    B, H, N, D = q.shape
    _check({"q": q}, q.shape, q.dtype, q.device)
    _check({"k": k, "v": v}, (B, hkv, N, D), q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check({"out": out}, q.shape, q.dtype, q.device)
    _check({"lse": lse}, (B, H, N), torch.float32, q.device)
    code = _dtype_code(q)
    if hkv != H:
        opt = opt if opt is not None else options()
        opt.h_kv = hkv
    if opt is None:
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, D, causal, scale, code, _stream_handle(q.device))
    else:
        need = fwd_ex_workspace_bytes(B, H, N, D, causal, code, opt)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws, wsb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None \
            else (None, 0)
        st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, H, N, D, causal, scale, code, opt, ws, wsb, _stream_handle(q.device))
    if st != FA_OK:
        raise FaError(st, what if opt is not None else "fa_fwd")
    return out, lse


def _bwd(q, k, v, o, lse, dout, causal, scale, opt, workspace, what):
    """Checks, allocations and one fa_bwd / fa_bwd_ex call; opt None = plain."""
    import torch
    hkv = _kv_heads(q, k)
    B, H, N, D = q.shape
    _check({"q": q, "o": o, "dout": dout}, q.shape, q.dtype, q.device)
    _check({"k": k, "v": v}, (B, hkv, N, D), q.dtype, q.device)
    _check({"lse": lse}, (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code = _dtype_code(q)
    if hkv != H:
        opt = opt if opt is not None else options()
        opt.h_kv = hkv
    need = bwd_ex_workspace_bytes(B, H, N, D, causal, code, opt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, causal, scale, code)
    wsa = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    st = fa_bwd(*args, *wsa) if opt is None else fa_bwd_ex(*args, opt, *wsa)
    if st != FA_OK:
        raise FaError(st, what if opt is not None else "fa_bwd")
    return dq, dk, dv


def _tiles_addr(tiles, B, N):
    if tiles is None:
        return 0
    if tiles.numel() < fa_mask_tiles_bytes(B, N):
        raise ValueError("tile table too small for B=%d N=%d" % (B, N))
    return tiles.data_ptr()


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """O, LSE = attention forward of fp16/bf16 device tensors q [B, H, N, D]
    and k, v [B, H_kv, N, D] (H_kv = H, or a divisor of H for grouped heads:
    fa_fwd_ex with fa_options.h_kv).

    Returns (o, lse) with o like q and lse float32 [B, H, N].
    """
    return _fwd(q, k, v, causal, scale, out, lse, None, None, "fa_fwd_ex")


def fwd_splitkv(q, k, v, num_splits=None, causal=False, scale=None, out=None, lse=None, workspace=None,
                dropout=None, tiles=None):
    """The forward with keys split into num_splits ranges and the partial
    states merged (fa_fwd_ex with fa_options.num_splits; None: the count of
    fa_fwd_splitkv_num_splits for the shape).  k, v may have fewer heads
    (grouped).  dropout=(p, seed, offset): the same result as fwd_dropout.
    tiles (from mask_tiles()): with a key-padding mask.  Returns (o, lse)."""
    B, H, N, D = q.shape
    if num_splits is None:
        num_splits = splitkv_num_splits(B, H, N, D, causal)
    opt = options(tiles=_tiles_addr(tiles, B, N), dropout=dropout, num_splits=num_splits)
    return _fwd(q, k, v, causal, scale, out, lse, opt, workspace, "fa_fwd_ex (split-K/V)")


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None):
    """dQ, dK, dV of the attention forward, by recomputation (dK, dV shaped
    like k, v: grouped heads get the sum over their query heads)."""
    return _bwd(q, k, v, o, lse, dout, causal, scale, None, workspace, "fa_bwd_ex")


def mask_tiles(key_mask):
    """Tile table (uint8 device tensor) of a [B, N] key-padding mask (bool or
    uint8 device tensor, nonzero = visible), built by fa_mask_tiles."""
    import torch
    if key_mask.dim() != 2 or not key_mask.is_cuda:
        raise ValueError("key_mask must be a [B, N] device tensor")
    m = key_mask.to(torch.uint8).contiguous()
    B, N = m.shape
    need = fa_mask_tiles_bytes(B, N)
    if need == 0:
        raise ValueError("unsupported mask shape %s" % (tuple(m.shape),))
    tiles = torch.empty(need, dtype=torch.uint8, device=m.device)
    st = fa_mask_tiles(m.data_ptr(), B, N, tiles.data_ptr(), need, _stream_handle(m.device))
    if st != FA_OK:
        raise FaError(st, "fa_mask_tiles")
    return tiles


def fwd_masked(q, k, v, tiles, causal=False, scale=None, out=None, lse=None):
    """The forward with a key-padding mask given by its tile table from
    mask_tiles() (fa_fwd_ex with fa_options.mask_tiles).  Returns (o, lse);
    rows with no visible key get o = 0 and lse = -inf."""
    B, H, N, D = q.shape
    opt = options(tiles=_tiles_addr(tiles, B, N))
    return _fwd(q, k, v, causal, scale, out, lse, opt, None, "fa_fwd_ex (mask)")


def bwd_masked(q, k, v, o, lse, dout, tiles, causal=False, scale=None, workspace=None):
    """Gradients of fwd_masked with the same tile table."""
    B, H, N, D = q.shape
    opt = options(tiles=_tiles_addr(tiles, B, N))
    return _bwd(q, k, v, o, lse, dout, causal, scale, opt, workspace, "fa_bwd_ex (mask)")


def fwd_dropout(q, k, v, dropout_p, seed, offset=0, causal=False, scale=None, out=None, lse=None, tiles=None):
    """The forward with attention dropout regenerated from (seed, offset)
    (fa_fwd_ex with fa_options.dropout).  k, v may have fewer heads
    (grouped); with tiles (from mask_tiles()) also a key-padding mask.
    Returns (o, lse)."""
    B, H, N, D = q.shape
    opt = options(tiles=_tiles_addr(tiles, B, N), dropout=(dropout_p, seed, offset))
    return _fwd(q, k, v, causal, scale, out, lse, opt, None, "fa_fwd_ex (dropout)")


def bwd_dropout(q, k, v, o, lse, dout, dropout_p, seed, offset=0, causal=False, scale=None, workspace=None,
                tiles=None):
    """Gradients of fwd_dropout with the same (p, seed, offset) and tile table."""
    B, H, N, D = q.shape
    opt = options(tiles=_tiles_addr(tiles, B, N), dropout=(dropout_p, seed, offset))
    return _bwd(q, k, v, o, lse, dout, causal, scale, opt, workspace, "fa_bwd_ex (dropout)")


def dropout_mask(B, H, N, dropout_p, seed, offset=0, device="cuda"):
    """The keep mask [B, H, N, N] (uint8, 1 = kept) of fwd_dropout / bwd_dropout."""
    import torch
    keep = torch.empty((B, H, N, N), dtype=torch.uint8, device=device)
    st = fa_dropout_mask(keep.data_ptr(), B, H, N, dropout_p, seed, offset, _stream_handle(keep.device))
    if st != FA_OK:
        raise FaError(st, "fa_dropout_mask")
    return keep
