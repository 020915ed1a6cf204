"""Thin Python binding of libsta (ctypes). Argument marshalling only.

Every function here checks tensor shapes, dtypes and devices, then calls the
C entry point of the same name with raw device pointers and the current HIP
stream. All arithmetic runs in the library's HIP kernels; there is no CPU or
PyTorch fallback: if libsta.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsta.so")

STA_OK, STA_ERR_INVALID_ARG, STA_ERR_UNSUPPORTED, STA_ERR_HIP = 0, -1, -2, -3
STA_BF16, STA_F32 = 0, 1
STA_MAX_HEADS = 256
ABI_VERSION = 7
STA_TILE_MAJOR, STA_RASTER = 0, 1

EXPORTS = (
    "sta_abi_version",
    "sta_reorder_tiles",
    "sta_restore_order",
    "sta_kv_tiles",
    "sta_q_tiles",
    "sta_tile_list_len",
    "sta_kv_pair_count",
    "sta_forward",
    "sta_forward_raster",
    "sta_forward_lse",
    "sta_forward_fp8",
    "sta_forward_fp8_lse",
    "sta_backward",
    "sta_backward_noalloc",
    "sta_window_recall",
    "sta_window_recall_fp8",
    "sta_full_attention",
    "sta_last_error",
)

_lib = None


class StaError(RuntimeError):
    """A HIP runtime error reported by libsta."""


def load_library(path: str = None) -> ctypes.CDLL:
    """Load libsta.so once and declare the C signatures.

    The default is the in-tree build; the STA_LIBRARY environment variable
    may name another build of the same library (e.g. a variant under test).
    """
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("STA_LIBRARY", LIB_PATH)
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Open one build of libsta at `path` and declare its C signatures
    (uncached: load_library keeps the one the binding uses)."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"libsta.so not found at {path}; build it with "
            "`python -m sparse_attention_video_tile_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_void_p, c_float = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    int3 = ctypes.POINTER(ctypes.c_int)
    lib.sta_abi_version.restype = c_int
    lib.sta_abi_version.argtypes = []
    lib.sta_last_error.restype = ctypes.c_char_p
    lib.sta_last_error.argtypes = []
    for name in ("sta_reorder_tiles", "sta_restore_order"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, int3, c_int, c_void_p]
    for name in ("sta_kv_tiles", "sta_q_tiles"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, int3, int3, c_int, c_void_p]
    lib.sta_forward_lse.restype = c_int
    lib.sta_forward_lse.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                    c_int, c_int, c_int, c_int, int3, int3, c_float, c_int, c_int,
                                    c_void_p]
    lib.sta_forward_fp8.restype = c_int
    lib.sta_forward_fp8.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                    c_int, c_int, c_int, int3, int3, c_float, c_float, c_float,
                                    c_int, c_void_p]
    lib.sta_forward_fp8_lse.restype = c_int
    lib.sta_forward_fp8_lse.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                        c_int, c_int, c_int, c_int, int3, int3, c_float, c_float,
                                        c_float, c_int, c_void_p]
    lib.sta_backward.restype = c_int
    lib.sta_backward.argtypes = [c_void_p] * 10 + [c_int, c_int, c_int, c_int, c_int, c_int, int3,
                                                   int3, c_float, c_int, c_int, c_void_p]
    lib.sta_backward_noalloc.restype = c_int
    lib.sta_backward_noalloc.argtypes = [c_void_p] * 9 + [c_int, c_int, c_int, c_int, c_int, c_int, int3,
                                                          int3, c_float, c_int, c_int, c_void_p]
    lib.sta_tile_list_len.restype = c_int
    lib.sta_tile_list_len.argtypes = [c_int, c_int, c_int, c_int, int3, int3, c_int]
    lib.sta_kv_pair_count.restype = ctypes.c_longlong
    lib.sta_kv_pair_count.argtypes = [c_int, c_int, c_int, c_int, int3, int3]
    for name in ("sta_forward", "sta_forward_raster"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                      c_int, c_int, c_int, int3, int3, c_float, c_int, c_void_p]
    lib.sta_window_recall_fp8.restype = c_int
    lib.sta_window_recall_fp8.argtypes = [c_void_p] * 4 + [c_int, c_int, c_int, c_int, c_int, c_int, int3,
                                                           c_void_p, c_int, c_float, c_float, c_float,
                                                           c_int, c_void_p]
    lib.sta_window_recall.restype = c_int
    lib.sta_window_recall.argtypes = [c_void_p] * 4 + [c_int, c_int, c_int, c_int, c_int, c_int, int3,
                                                       int3, c_int, c_float, c_int, c_int, c_void_p]
    lib.sta_full_attention.restype = c_int
    lib.sta_full_attention.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                       c_int, c_int, c_float, c_int, c_void_p]
    if lib.sta_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libsta ABI {lib.sta_abi_version()} != expected {ABI_VERSION}")
    return lib


def last_error() -> str:
    return load_library().sta_last_error().decode()


def _check(rc: int, what: str) -> None:
    if rc == STA_OK:
        return
    msg = f"{what}: {last_error()}"
    if rc == STA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if rc == STA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise StaError(msg)


def _int_array(values: Sequence[int]):
    flat = [int(x) for x in values]
    return (ctypes.c_int * len(flat))(*flat)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return STA_BF16
    if t.dtype == torch.float32:
        return STA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _require_gpu(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU device")
        if t.device != dev:
            raise ValueError("tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def tile_major_rows(volume: Sequence[int], tile: Sequence[int]) -> int:
    """Rows of a tile-major tensor: n_tiles * tau, with n = ceil(extent / c) per
    axis (a volume the tile does not divide is padded up to whole tiles)."""
    rows = 1
    for e, c in zip(volume, tile):
        rows *= -(-int(e) // int(c)) * int(c)
    return rows


def _windows_per_head(window, heads: int):
    w = torch.as_tensor(window, dtype=torch.int64).reshape(-1, 3)
    if w.shape[0] == 1 and heads > 1:
        w = w.expand(heads, 3)
    if w.shape[0] != heads:
        raise ValueError(f"need one window per head ({heads}) or one for all; got {w.shape[0]}")
    return [int(x) for x in w.reshape(-1).tolist()]


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def sta_reorder_tiles(x: torch.Tensor, tile: Sequence[int], out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Raster (B, heads, T, H, W, d) -> tile-major (B, heads, n_tiles * tau, d);
    padding rows of a volume the tile does not divide are zeros."""
    lib = load_library()
    if x.dim() != 6:
        raise ValueError("x must be (B, heads, T, H, W, d)")
    B, heads, T, H, W, d = x.shape
    rows = tile_major_rows((T, H, W), tile)
    if out is None:
        out = torch.empty((B, heads, rows, d), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, heads, rows, d) or out.dtype != x.dtype:
        raise ValueError("out must be (B, heads, S, d) with the input's dtype")
    dev = _require_gpu(x, out)
    with torch.cuda.device(dev):
        rc = lib.sta_reorder_tiles(x.data_ptr(), out.data_ptr(), B, heads, d, T, H, W,
                                   _int_array(tile), _dtype_code(x), _stream(dev))
    _check(rc, "sta_reorder_tiles")
    return out


def sta_restore_order(x: torch.Tensor, volume: Sequence[int], tile: Sequence[int],
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tile-major (B, heads, S, d) -> raster (B, heads, T, H, W, d)."""
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be (B, heads, S, d)")
    B, heads, S, d = x.shape
    T, H, W = (int(a) for a in volume)
    if S != tile_major_rows(volume, tile):
        raise ValueError(f"S={S} does not match volume {tuple(volume)} with tile {tuple(tile)}")
    if out is None:
        out = torch.empty((B, heads, T, H, W, d), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, heads, T, H, W, d) or out.dtype != x.dtype:
        raise ValueError("out must be (B, heads, T, H, W, d) with the input's dtype")
    dev = _require_gpu(x, out)
    with torch.cuda.device(dev):
        rc = lib.sta_restore_order(x.data_ptr(), out.data_ptr(), B, heads, d, T, H, W,
                                   _int_array(tile), _dtype_code(x), _stream(dev))
    _check(rc, "sta_restore_order")
    return out


def sta_kv_pair_count(heads: int, volume: Sequence[int], tile: Sequence[int], window) -> int:
    """Computed (query tile, key tile) pairs summed over heads (host only)."""
    lib = load_library()
    T, H, W = (int(a) for a in volume)
    n = lib.sta_kv_pair_count(heads, T, H, W, _int_array(tile),
                              _int_array(_windows_per_head(window, heads)))
    if n < 0:
        _check(int(n), "sta_kv_pair_count")
    return int(n)


def sta_tile_list_len(heads: int, volume: Sequence[int], tile: Sequence[int], window,
                      transposed: bool = False) -> int:
    """Longest list of sta_kv_tiles (transposed=False) or sta_q_tiles
    (transposed=True), computed by the library (host only)."""
    lib = load_library()
    T, H, W = (int(a) for a in volume)
    n = lib.sta_tile_list_len(heads, T, H, W, _int_array(tile),
                              _int_array(_windows_per_head(window, heads)), int(bool(transposed)))
    if n < 0:
        _check(int(n), "sta_tile_list_len")
    return int(n)


def _tile_lists(fn_name: str, heads: int, volume, tile, window, max_len, device, transposed: bool):
    lib = load_library()
    T, H, W = (int(a) for a in volume)
    ws = _windows_per_head(window, heads)
    n_tiles = tile_major_rows(volume, tile) // (int(tile[0]) * int(tile[1]) * int(tile[2]))
    if max_len is None:
        max_len = sta_tile_list_len(heads, volume, tile, ws, transposed)
    lists = torch.empty((heads, n_tiles, max_len), dtype=torch.int32, device=device)
    counts = torch.empty((heads, n_tiles), dtype=torch.int32, device=device)
    dev = _require_gpu(lists, counts)
    with torch.cuda.device(dev):
        rc = getattr(lib, fn_name)(lists.data_ptr(), counts.data_ptr(), heads, T, H, W,
                                   _int_array(tile), _int_array(ws), max_len, _stream(dev))
    _check(rc, fn_name)
    return lists, counts


def sta_kv_tiles(heads: int, volume: Sequence[int], tile: Sequence[int], window,
                 max_kv: Optional[int] = None, device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    """Per head and query tile, the window's key tiles (ascending) and their count."""
    return _tile_lists("sta_kv_tiles", heads, volume, tile, window, max_kv, device, False)


def sta_q_tiles(heads: int, volume: Sequence[int], tile: Sequence[int], window,
                max_q: Optional[int] = None, device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    """Per head and key tile, the query tiles whose window holds it (ascending) and their count."""
    return _tile_lists("sta_q_tiles", heads, volume, tile, window, max_q, device, True)


def sta_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, volume: Sequence[int],
                tile: Sequence[int], window, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """STA forward on tile-major (B, heads, S, d) tensors; returns tile-major output."""
    lib = load_library()
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be (B, heads, S, d)")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, heads, S, d = q.shape
    T, H, W = (int(a) for a in volume)
    if S != tile_major_rows(volume, tile):
        raise ValueError(f"S={S} does not match volume {tuple(volume)} with tile {tuple(tile)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    dev = _require_gpu(q, k, v, out)
    with torch.cuda.device(dev):
        rc = lib.sta_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, heads, d,
                             T, H, W, _int_array(tile), _int_array(_windows_per_head(window, heads)),
                             float(scale), _dtype_code(q), _stream(dev))
    _check(rc, "sta_forward")
    return out


def sta_full_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense softmax attention over all S keys; (B, heads, S, d) in any token order."""
    lib = load_library()
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be (B, heads, S, d)")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, heads, S, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    dev = _require_gpu(q, k, v, out)
    with torch.cuda.device(dev):
        rc = lib.sta_full_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                    heads, d, S, float(scale), _dtype_code(q), _stream(dev))
    _check(rc, "sta_full_attention")
    return out


def sta_forward_raster(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tile: Sequence[int],
                       window, scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """STA forward on raster (B, heads, T, H, W, d) tensors in one kernel;
    returns the raster-order output (same values as reorder, sta_forward,
    restore)."""
    lib = load_library()
    if q.dim() != 6 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be (B, heads, T, H, W, d)")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    B, heads, T, H, W, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    dev = _require_gpu(q, k, v, out)
    with torch.cuda.device(dev):
        rc = lib.sta_forward_raster(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                    heads, d, T, H, W, _int_array(tile),
                                    _int_array(_windows_per_head(window, heads)), float(scale),
                                    _dtype_code(q), _stream(dev))
    _check(rc, "sta_forward_raster")
    return out


def _order_shapes(q: torch.Tensor, volume, tile):
    """(B, heads, d, (T, H, W), order code) of a raster 6-D or tile-major 4-D tensor."""
    if q.dim() == 6:
        B, heads, T, H, W, d = q.shape
        return B, heads, d, (T, H, W), STA_RASTER
    if q.dim() == 4:
        if volume is None:
            raise ValueError("tile-major (B, heads, S, d) tensors need the volume")
        B, heads, S, d = q.shape
        T, H, W = (int(a) for a in volume)
        if S != tile_major_rows(volume, tile):
            raise ValueError(f"S={S} does not match volume {tuple(volume)} with tile {tuple(tile)}")
        return B, heads, d, (T, H, W), STA_TILE_MAJOR
    raise ValueError("tensors must be raster (B, heads, T, H, W, d) or tile-major (B, heads, S, d)")


def sta_forward_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tile: Sequence[int], window,
                    scale: Optional[float] = None, volume: Optional[Sequence[int]] = None,
                    out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """STA forward returning (out, lse). Raster (B, heads, T, H, W, d) tensors,
    or tile-major (B, heads, S, d) ones with `volume`; lse is float32 of the
    tensors' shape without d."""
    lib = load_library()
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    B, heads, d, (T, H, W), order = _order_shapes(q, volume, tile)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    elif lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of q's shape without d")
    dev = _require_gpu(q, k, v, out, lse)
    with torch.cuda.device(dev):
        rc = lib.sta_forward_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, heads, d, T, H, W, _int_array(tile),
                                 _int_array(_windows_per_head(window, heads)), float(scale),
                                 _dtype_code(q), order, _stream(dev))
    _check(rc, "sta_forward_lse")
    return out, lse


_FP8_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def sta_forward_fp8(q8: torch.Tensor, k8: torch.Tensor, v: torch.Tensor, tile: Sequence[int], window,
                    q_descale: float, k_descale: float, scale: Optional[float] = None,
                    volume: Optional[Sequence[int]] = None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """STA forward with fp8 (OCP E4M3) q8, k8 (torch.uint8 codes or
    torch.float8_e4m3fn), per-tensor descales and bf16 v; returns bf16 out.
    Raster (B, heads, T, H, W, 128) tensors, or tile-major (B, heads, S, 128)
    ones with `volume`."""
    return _forward_fp8(q8, k8, v, tile, window, q_descale, k_descale, scale, volume, out, None, False)


def sta_forward_fp8_lse(q8: torch.Tensor, k8: torch.Tensor, v: torch.Tensor, tile: Sequence[int],
                        window, q_descale: float, k_descale: float, scale: Optional[float] = None,
                        volume: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """sta_forward_fp8 returning (out, lse); lse is float32 of v's shape
    without d, the row log-sum-exp of the scores on the decoded values."""
    return _forward_fp8(q8, k8, v, tile, window, q_descale, k_descale, scale, volume, out, lse, True)


def _forward_fp8(q8, k8, v, tile, window, q_descale, k_descale, scale, volume, out, lse, with_lse):
    lib = load_library()
    if q8.shape != k8.shape or q8.shape != v.shape:
        raise ValueError("q8, k8, v must share a shape")
    if q8.dtype not in _FP8_DTYPES or k8.dtype not in _FP8_DTYPES:
        raise TypeError("q8 and k8 must be torch.uint8 codes or torch.float8_e4m3fn")
    if v.dtype != torch.bfloat16:
        raise TypeError("v must be torch.bfloat16")
    B, heads, d, (T, H, W), order = _order_shapes(v, volume, tile)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(v)
    elif out.shape != v.shape or out.dtype != v.dtype:
        raise ValueError("out must match v")
    if not with_lse:
        dev = _require_gpu(q8, k8, v, out)
        with torch.cuda.device(dev):
            rc = lib.sta_forward_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                     heads, d, T, H, W, _int_array(tile),
                                     _int_array(_windows_per_head(window, heads)), float(scale),
                                     float(q_descale), float(k_descale), order, _stream(dev))
        _check(rc, "sta_forward_fp8")
        return out
    if lse is None:
        lse = torch.empty(v.shape[:-1], dtype=torch.float32, device=v.device)
    elif lse.shape != v.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of v's shape without d")
    dev = _require_gpu(q8, k8, v, out, lse)
    with torch.cuda.device(dev):
        rc = lib.sta_forward_fp8_lse(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, heads, d, T, H, W, _int_array(tile),
                                     _int_array(_windows_per_head(window, heads)), float(scale),
                                     float(q_descale), float(k_descale), order, _stream(dev))
    _check(rc, "sta_forward_fp8_lse")
    return out, lse


def sta_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                 dout: torch.Tensor, lse: torch.Tensor, tile: Sequence[int], window,
                 scale: Optional[float] = None, volume: Optional[Sequence[int]] = None,
                 delta: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of sum(dout * out) for out = STA(q, k, v), from
    the forward's out and lse. Same token order conventions as sta_forward_lse;
    `delta` is an optional float32 workspace shaped like lse."""
    lib = load_library()
    for name, x in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, heads, d, (T, H, W), order = _order_shapes(q, volume, tile)
    if lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of q's shape without d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if delta is None:
        delta = torch.empty_like(lse)
    elif delta.shape != lse.shape or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 tensor shaped like lse")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dev = _require_gpu(q, k, v, out, dout, lse, delta, dq, dk, dv)
    with torch.cuda.device(dev):
        rc = lib.sta_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), delta.data_ptr(), B, heads, d, T, H, W,
                              _int_array(tile), _int_array(_windows_per_head(window, heads)),
                              float(scale), _dtype_code(q), order, _stream(dev))
    _check(rc, "sta_backward")
    return dq, dk, dv


def sta_backward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                         dout: torch.Tensor, lse: torch.Tensor, tile: Sequence[int], window,
                         scale: Optional[float] = None, volume: Optional[Sequence[int]] = None,
                         grads: Optional[Sequence[torch.Tensor]] = None
                         ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """sta_backward through the library's allocation-free entry point (its D
    workspace is a static device array; calls that overlap on one GPU race).
    `grads` may supply the (dq, dk, dv) output tensors."""
    lib = load_library()
    for name, x in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, heads, d, (T, H, W), order = _order_shapes(q, volume, tile)
    if lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of q's shape without d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    dq, dk, dv = grads
    for x in grads:
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError("gradient outputs must match q in shape and dtype")
    dev = _require_gpu(q, k, v, out, dout, lse, dq, dk, dv)
    with torch.cuda.device(dev):
        rc = lib.sta_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), B, heads, d, T, H, W, _int_array(tile),
                                      _int_array(_windows_per_head(window, heads)), float(scale),
                                      _dtype_code(q), order, _stream(dev))
    _check(rc, "sta_backward_noalloc")
    return dq, dk, dv


def sta_window_recall(q: torch.Tensor, k: torch.Tensor, tile: Sequence[int], candidates,
                      scale: Optional[float] = None, volume: Optional[Sequence[int]] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Share of full-attention probability each candidate window keeps, averaged
    over the query rows: float32 (B, heads, n_candidates). Raster 6-D tensors,
    or tile-major 4-D ones with `volume`. `workspace` (float32, (n_candidates +
    1) * B * heads * S elements) receives the row log-sum-exps: all keys, then
    each candidate's window."""
    lib = load_library()
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("k must match q in shape and dtype")
    B, heads, d, (T, H, W), order = _order_shapes(q, volume, tile)
    cand = [int(x) for x in torch.as_tensor(candidates, dtype=torch.int64).reshape(-1).tolist()]
    if len(cand) == 0 or len(cand) % 3:
        raise ValueError("candidates must be a non-empty list of (t, h, w) windows")
    n = len(cand) // 3
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = T * H * W if order == STA_RASTER else tile_major_rows((T, H, W), tile)
    if workspace is None:
        workspace = torch.empty((n + 1, B, heads, S), dtype=torch.float32, device=q.device)
    elif (workspace.numel() < (n + 1) * B * heads * S or workspace.dtype != torch.float32
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous float32 tensor of at least "
                         "(n_candidates+1)*B*heads*S elements")
    recall = torch.empty((B, heads, n), dtype=torch.float32, device=q.device)
    dev = _require_gpu(q, k, recall, workspace)
    with torch.cuda.device(dev):
        rc = lib.sta_window_recall(q.data_ptr(), k.data_ptr(), recall.data_ptr(), workspace.data_ptr(),
                                   B, heads, d, T, H, W, _int_array(tile), _int_array(cand), n,
                                   float(scale), _dtype_code(q), order, _stream(dev))
    _check(rc, "sta_window_recall")
    return recall


def sta_window_recall_fp8(q8: torch.Tensor, k8: torch.Tensor, tile: Sequence[int], candidates,
                          q_descale: float, k_descale: float, scale: Optional[float] = None,
                          volume: Optional[Sequence[int]] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sta_window_recall on fp8 (OCP E4M3) q8, k8 (torch.uint8 codes or
    torch.float8_e4m3fn) with per-tensor descales: float32 (B, heads,
    n_candidates)."""
    lib = load_library()
    if k8.shape != q8.shape:
        raise ValueError("k8 must match q8 in shape")
    if q8.dtype not in _FP8_DTYPES or k8.dtype not in _FP8_DTYPES:
        raise TypeError("q8 and k8 must be torch.uint8 codes or torch.float8_e4m3fn")
    B, heads, d, (T, H, W), order = _order_shapes(q8, volume, tile)
    cand = [int(x) for x in torch.as_tensor(candidates, dtype=torch.int64).reshape(-1).tolist()]
    if len(cand) == 0 or len(cand) % 3:
        raise ValueError("candidates must be a non-empty list of (t, h, w) windows")
    n = len(cand) // 3
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = T * H * W if order == STA_RASTER else tile_major_rows((T, H, W), tile)
    if workspace is None:
        workspace = torch.empty((n + 1, B, heads, S), dtype=torch.float32, device=q8.device)
    elif (workspace.numel() < (n + 1) * B * heads * S or workspace.dtype != torch.float32
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous float32 tensor of at least "
                         "(n_candidates+1)*B*heads*S elements")
    recall = torch.empty((B, heads, n), dtype=torch.float32, device=q8.device)
    dev = _require_gpu(q8, k8, recall, workspace)
    with torch.cuda.device(dev):
        rc = lib.sta_window_recall_fp8(q8.data_ptr(), k8.data_ptr(), recall.data_ptr(),
                                       workspace.data_ptr(), B, heads, d, T, H, W, _int_array(tile),
                                       _int_array(cand), n, float(scale), float(q_descale),
                                       float(k_descale), order, _stream(dev))
    _check(rc, "sta_window_recall_fp8")
    return recall


class _STAFunction(torch.autograd.Function):
    """Autograd wrapper: forward via sta_forward_lse, backward via sta_backward."""

    @staticmethod
    def forward(ctx, q, k, v, tile, window, scale, volume):
        out, lse = sta_forward_lse(q, k, v, tile, window, scale, volume)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.cfg = (tuple(tile), window, scale, volume)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        tile, window, scale, volume = ctx.cfg
        dq, dk, dv = sta_backward(q, k, v, out, dout.contiguous(), lse, tile, window, scale, volume)
        return dq, dk, dv, None, None, None, None


def sta_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tile: Sequence[int], window,
                  scale: Optional[float] = None, volume: Optional[Sequence[int]] = None) -> torch.Tensor:
    """STA as a differentiable torch op (raster 6-D tensors, or tile-major 4-D
    ones with `volume`); gradients come from sta_backward."""
    return _STAFunction.apply(q.contiguous(), k.contiguous(), v.contiguous(), tile, window, scale, volume)


def sliding_tile_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tile: Sequence[int],
                           window, scale: Optional[float] = None, fused: bool = True) -> torch.Tensor:
    """The whole path on raster (B, heads, T, H, W, d) tensors. fused=True runs
    the single raster-order kernel; when the library has no raster-order
    kernel for the request (it refuses with STA_ERR_UNSUPPORTED, e.g. a window
    run longer than its offset table) or fused=False, q, k, v are reordered to
    tile-major, STA forward runs, and the output is restored to raster order.
    Both give the same values."""
    if q.dim() != 6:
        raise ValueError("q, k, v must be (B, heads, T, H, W, d)")
    if fused:
        try:
            return sta_forward_raster(q, k, v, tile, window, scale)
        except NotImplementedError:
            pass
    volume = tuple(q.shape[2:5])
    qt, kt, vt = (sta_reorder_tiles(x, tile) for x in (q, k, v))
    ot = sta_forward(qt, kt, vt, volume, tile, window, scale)
    return sta_restore_order(ot, volume, tile)
