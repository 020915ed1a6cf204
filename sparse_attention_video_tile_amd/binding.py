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
ABI_VERSION = 2
# Longest window run (omega_w * tau keys) sta_forward_raster accepts.
STA_MAX_RASTER_RUN = 8192

EXPORTS = (
    "sta_abi_version",
    "sta_reorder_tiles",
    "sta_restore_order",
    "sta_kv_tiles",
    "sta_kv_pair_count",
    "sta_forward",
    "sta_forward_raster",
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
    lib.sta_kv_tiles.restype = c_int
    lib.sta_kv_tiles.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, int3, int3, c_int, c_void_p]
    lib.sta_kv_pair_count.restype = ctypes.c_longlong
    lib.sta_kv_pair_count.argtypes = [c_int, c_int, c_int, c_int, int3, int3]
    for name in ("sta_forward", "sta_forward_raster"):
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                      c_int, c_int, c_int, int3, int3, c_float, c_int, c_void_p]
    lib.sta_full_attention.restype = c_int
    lib.sta_full_attention.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                       c_int, c_int, c_float, c_int, c_void_p]
    if lib.sta_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libsta ABI {lib.sta_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
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
    """Raster (B, heads, T, H, W, d) -> tile-major (B, heads, S, d)."""
    lib = load_library()
    if x.dim() != 6:
        raise ValueError("x must be (B, heads, T, H, W, d)")
    B, heads, T, H, W, d = x.shape
    if out is None:
        out = torch.empty((B, heads, T * H * W, d), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, heads, T * H * W, d) or out.dtype != x.dtype:
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
    if S != T * H * W:
        raise ValueError(f"S={S} does not match volume {tuple(volume)}")
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


def sta_kv_tiles(heads: int, volume: Sequence[int], tile: Sequence[int], window,
                 max_kv: Optional[int] = None, device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    """Per head and query tile, the window's key tiles (ascending) and their count."""
    lib = load_library()
    T, H, W = (int(a) for a in volume)
    ws = _windows_per_head(window, heads)
    n_tiles = (T // int(tile[0])) * (H // int(tile[1])) * (W // int(tile[2]))
    if max_kv is None:
        max_kv = max(
            (ws[3 * h] // int(tile[0])) * (ws[3 * h + 1] // int(tile[1])) * (ws[3 * h + 2] // int(tile[2]))
            for h in range(heads))
    kv_list = torch.empty((heads, n_tiles, max_kv), dtype=torch.int32, device=device)
    kv_count = torch.empty((heads, n_tiles), dtype=torch.int32, device=device)
    dev = _require_gpu(kv_list, kv_count)
    with torch.cuda.device(dev):
        rc = lib.sta_kv_tiles(kv_list.data_ptr(), kv_count.data_ptr(), heads, T, H, W,
                              _int_array(tile), _int_array(ws), max_kv, _stream(dev))
    _check(rc, "sta_kv_tiles")
    return kv_list, kv_count


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
    if S != T * H * W:
        raise ValueError(f"S={S} does not match volume {tuple(volume)}")
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


def raster_run_fits(tile: Sequence[int], window, heads: int) -> bool:
    """Whether every head's window run (omega_w * tau keys) is within what
    sta_forward_raster accepts."""
    ws = _windows_per_head(window, heads)
    tau = int(tile[0]) * int(tile[1]) * int(tile[2])
    return all((ws[3 * h + 2] // int(tile[2])) * tau <= STA_MAX_RASTER_RUN for h in range(heads))


def sliding_tile_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tile: Sequence[int],
                           window, scale: Optional[float] = None, fused: bool = True) -> torch.Tensor:
    """The whole path on raster (B, heads, T, H, W, d) tensors. fused=True runs
    the single raster-order kernel when the windows allow it; otherwise q, k, v
    are reordered to tile-major, STA forward runs, and the output is restored
    to raster order. Both give the same values."""
    if q.dim() != 6:
        raise ValueError("q, k, v must be (B, heads, T, H, W, d)")
    if fused and raster_run_fits(tile, window, q.shape[1]):
        return sta_forward_raster(q, k, v, tile, window, scale)
    volume = tuple(q.shape[2:5])
    qt, kt, vt = (sta_reorder_tiles(x, tile) for x in (q, k, v))
    ot = sta_forward(qt, kt, vt, volume, tile, window, scale)
    return sta_restore_order(ot, volume, tile)
