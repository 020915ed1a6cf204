"""CPU oracle for Sliding Tile Attention (STA) forward -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module. It shares no code with the HIP library and never calls it.

What STA computes (sources are the pages on "Fast Video Generation with Sliding
Tile Attention"):

* The latent video is a (T, H, W) grid of tokens. A tile is a contiguous
  (c_t, c_h, c_w) cube of tokens (hotaipapers podcast transcript, the answer on
  what a tile is; dianyo ICML2025 blog, STA "Observation & Proposed Method").
* The window slides tile by tile: every query in one tile attends to the same
  keys, namely the tokens of the key tiles inside the tile's local 3D window
  (same two passages; neuronad article, "Enter Sliding Tile Attention").
* Consequently each (query tile, key tile) block of the attention map is either
  wholly kept or wholly skipped; there are no mixed blocks (podcast, the answer
  on dense / empty / mixed blocks; atlas.scime.ai summary, "Approach").
* Windows are given per head as token triples such as (18,24,24) and
  (30,40,40) (atlas.scime.ai summary, measured-effects table).

Readings taken where the pages are silent:

* Boundary: the window keeps its full size and its centre is clamped so that
  the window stays inside the volume. Per axis a, with query tile coordinate
  q_a, n_a tiles and a window of w_a tiles,
      start_a = min(max(q_a - floor(w_a / 2), 0), n_a - w_a),
  and the window covers key tiles start_a .. start_a + w_a - 1. The pages'
  91% sparsity for (18,24,24) (atlas.scime.ai summary, "Key results") is what
  this rule gives on the 30x48x80 volume with (6,8,8) tiles.
* Softmax is base e with a positive scale (1/sqrt(d) by default).
* Tile-major order: tiles in raster (t, h, w) order, tokens inside a tile in
  raster order.
* A volume the tile does not divide is covered by the grid of ceil(extent /
  c) tiles per axis, as if padded up to whole tiles; windows are counted in
  tiles of that grid with the same rule. Padded positions are not tokens:
  they are never keys and have no output. Tile-major tensors of such a volume
  hold n_tiles * tau rows, the padded positions as zero rows.

All arithmetic here is float64. The attention is the plain definition: an
explicit token-level mask built from token coordinates, then a two-pass
softmax (max, then exp and normalise) over the allowed keys.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

Triple = Tuple[int, int, int]


# ----------------------------------------------------------------------------
# Window geometry
# ----------------------------------------------------------------------------

def tile_grid(volume: Sequence[int], tile: Sequence[int]) -> Triple:
    """Number of tiles per axis, n_a = ceil(extent_a / c_a) (the last tile of an
    axis the tile does not divide is partly padding)."""
    n = []
    for e, c in zip(volume, tile):
        if c <= 0 or e <= 0:
            raise ValueError(f"tile {tuple(tile)} and volume {tuple(volume)} must be positive")
        n.append(-(-e // c))
    return tuple(n)


def is_padded(volume: Sequence[int], tile: Sequence[int]) -> bool:
    return any(e % c for e, c in zip(volume, tile))


def window_in_tiles(window: Sequence[int], tile: Sequence[int], volume: Sequence[int]) -> Triple:
    """Window size in tiles, w_a / c_a; the window must be whole tiles within the
    tile grid (at most n_a tiles)."""
    out = []
    n = tile_grid(volume, tile)
    for w, c, na in zip(window, tile, n):
        if w <= 0 or w % c or w // c > na:
            raise ValueError(f"window {tuple(window)} is not whole tiles of {tuple(tile)} within {tuple(volume)}")
        out.append(w // c)
    return tuple(out)


def window_start(q_tile: int, n: int, omega: int) -> int:
    """First key tile of the clamped window along one axis."""
    return min(max(q_tile - omega // 2, 0), n - omega)


# ----------------------------------------------------------------------------
# Token-level mask
# ----------------------------------------------------------------------------

def token_coords(volume: Sequence[int]) -> np.ndarray:
    """(S, 3) integer coordinates (t, y, x) of every token in raster order."""
    T, H, W = volume
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)


def axis_mask(extent: int, c: int, omega: int) -> np.ndarray:
    """Per-axis mask A[r, r']: may a query at coordinate r see a key at r' along this axis.

    The query's tile is floor(r / c); its window starts at the clamped start
    and spans ``omega`` tiles; the key is inside iff its own tile floor(r'/c)
    lies in that span.
    """
    n = -(-extent // c)
    r = np.arange(extent)
    start = np.array([window_start(int(x) // c, n, omega) for x in r])
    k_tile = r // c
    return (k_tile[None, :] >= start[:, None]) & (k_tile[None, :] < start[:, None] + omega)


def token_mask_rows(volume, tile, window, query_tokens: np.ndarray) -> np.ndarray:
    """Boolean mask M[r, j]: may query token ``query_tokens[r]`` (raster index) see key token j.

    A key is visible iff it is inside the window along every axis; each query
    and key token is placed by its own coordinates.
    """
    tile_grid(volume, tile)
    om = window_in_tiles(window, tile, volume)
    T, H, W = volume
    qc = token_coords(volume)[np.asarray(query_tokens)]  # (R, 3)
    at, ah, aw = (axis_mask(volume[a], tile[a], om[a])[qc[:, a]] for a in range(3))  # (R, extent_a)
    # key token (t, y, x) is visible iff it is inside along t AND y AND x;
    # the key axis is raster order, so the (R, T, H, W) AND flattens to (R, S)
    allowed = at[:, :, None, None] & ah[:, None, :, None] & aw[:, None, None, :]
    return allowed.reshape(qc.shape[0], T * H * W)


def tile_tokens(volume, tile, tile_index: int) -> np.ndarray:
    """Raster indices of the tokens of tile ``tile_index`` (tiles in raster order)."""
    T, H, W = volume
    n = tile_grid(volume, tile)
    it, rem = divmod(tile_index, n[1] * n[2])
    ih, iw = divmod(rem, n[2])
    # positions past the volume (a partly padded tile) are not tokens
    t = np.arange(it * tile[0], min((it + 1) * tile[0], T))
    y = np.arange(ih * tile[1], min((ih + 1) * tile[1], H))
    x = np.arange(iw * tile[2], min((iw + 1) * tile[2], W))
    tt, yy, xx = np.meshgrid(t, y, x, indexing="ij")
    return ((tt * H + yy) * W + xx).ravel()


def _classify_blocks(mask: np.ndarray, cq: int, ck: int) -> np.ndarray:
    """Split a 2-D mask into (cq x ck) blocks; True = all kept, False = all skipped.

    Raises on a block that is partly kept (a mixed block).
    """
    R, C = mask.shape
    blocks = mask.reshape(R // cq, cq, C // ck, ck)
    full = blocks.all(axis=(1, 3))
    empty = ~blocks.any(axis=(1, 3))
    mixed = ~(full | empty)
    if mixed.any():
        i, j = np.argwhere(mixed)[0]
        raise AssertionError(f"mixed block at query block {i}, key block {j}")
    return full


def tile_selection(volume, tile, window) -> np.ndarray:
    """Boolean (N_t, N_t) matrix: key tile j is computed for query tile i.

    The token mask is the AND of one mask per axis, so the (tile i) x (tile j)
    block of the token mask is the outer AND of one (c_a x c_a) block per axis.
    Each per-axis block must be all kept or all skipped (else the 3-D block is
    mixed, which raises); the 3-D block is then kept iff all three are kept.
    """
    n = tile_grid(volume, tile)
    om = window_in_tiles(window, tile, volume)
    # The rule applied to every position of the tile grid (padded ones too)
    # gives whole blocks; on a divisible volume these are exactly the token
    # mask's blocks.
    per_axis = [
        _classify_blocks(axis_mask(n[a] * tile[a], tile[a], om[a]), tile[a], tile[a]) for a in range(3)
    ]
    sel = (per_axis[0][:, None, None, :, None, None]
           & per_axis[1][None, :, None, None, :, None]
           & per_axis[2][None, None, :, None, None, :])
    n_tiles = n[0] * n[1] * n[2]
    return sel.reshape(n_tiles, n_tiles)


def tile_selection_from_token_mask(volume, tile, window) -> np.ndarray:
    """Same as :func:`tile_selection`, from the full 3-D token mask (small,
    tile-divisible volumes only)."""
    if is_padded(volume, tile):
        raise ValueError("needs a volume the tile divides")
    n = tile_grid(volume, tile)
    n_tiles = n[0] * n[1] * n[2]
    S = volume[0] * volume[1] * volume[2]
    tau = tile[0] * tile[1] * tile[2]
    order = np.concatenate([tile_tokens(volume, tile, j) for j in range(n_tiles)])
    mask = token_mask_rows(volume, tile, window, order)[:, order]  # both axes tile-major
    assert mask.shape == (S, S)
    return _classify_blocks(mask, tau, tau)


def kv_tile_lists(volume, tile, windows: np.ndarray, max_kv: int | None = None):
    """Per head and query tile: the selected key tiles in ascending tile index.

    Returns (lists int32 [heads, N_t, max_kv] padded with -1, counts int32 [heads, N_t]).
    Ascending tile index is raster (t, h, w) order of tile coordinates.
    """
    windows = np.asarray(windows).reshape(-1, 3)
    sels = [tile_selection(volume, tile, tuple(int(x) for x in w)) for w in windows]
    n_tiles = sels[0].shape[0]
    counts = np.stack([s.sum(axis=1) for s in sels]).astype(np.int32)
    if max_kv is None:
        max_kv = int(counts.max())
    lists = np.full((len(sels), n_tiles, max_kv), -1, dtype=np.int32)
    for h, s in enumerate(sels):
        for i in range(n_tiles):
            idx = np.nonzero(s[i])[0]
            lists[h, i, : len(idx)] = idx
    return lists, counts


def kv_pair_count(volume, tile, windows: np.ndarray) -> int:
    """Number of computed (query tile, key tile) pairs summed over heads."""
    return int(sum(tile_selection(volume, tile, tuple(int(x) for x in w)).sum()
                   for w in np.asarray(windows).reshape(-1, 3)))


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def _masked_softmax_attention(q_rows, k_all, v_all, allowed, scale):
    """Two-pass softmax attention of query rows over the keys they may see (float64)."""
    s = scale * (q_rows @ k_all.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise AssertionError("a query row sees no key")
    p = np.where(allowed, np.exp(s - m), 0.0)
    return (p @ v_all) / p.sum(axis=1, keepdims=True)


def sta_attention_rows(q, k, v, tile, window, scale, b: int, h: int, query_tokens) -> np.ndarray:
    """STA output rows for batch ``b``, head ``h`` and the given raster query tokens.

    q, k, v: (B, heads, T, H, W, d) arrays in raster token order.
    Returns float64 (len(query_tokens), d).
    """
    volume = q.shape[2:5]
    d = q.shape[-1]
    qf = np.asarray(q[b, h], dtype=np.float64).reshape(-1, d)
    kf = np.asarray(k[b, h], dtype=np.float64).reshape(-1, d)
    vf = np.asarray(v[b, h], dtype=np.float64).reshape(-1, d)
    qt = np.asarray(query_tokens)
    allowed = token_mask_rows(volume, tile, window, qt)
    return _masked_softmax_attention(qf[qt], kf, vf, allowed, scale)


def sta_attention(q, k, v, tile, windows, scale) -> np.ndarray:
    """Full STA output in raster order, float64, shape (B, heads, T, H, W, d).

    Query rows are processed one tile at a time to bound memory; the mask of
    each row still comes from that row's own coordinates.
    """
    B, heads = q.shape[:2]
    volume = q.shape[2:5]
    d = q.shape[-1]
    windows = np.asarray(windows).reshape(heads, 3)
    n = tile_grid(volume, tile)
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            of = out[b, h].reshape(-1, d)
            w = tuple(int(x) for x in windows[h])
            for i in range(n[0] * n[1] * n[2]):
                rows = tile_tokens(volume, tile, i)
                of[rows] = sta_attention_rows(q, k, v, tile, w, scale, b, h, rows)
    return out


def full_attention(q, k, v, scale) -> np.ndarray:
    """Plain softmax attention of every token over every token, float64.

    q, k, v: (B, heads, S, d) or (B, heads, T, H, W, d).
    """
    shape = q.shape
    d = shape[-1]
    B, heads = shape[:2]
    qf = np.asarray(q, dtype=np.float64).reshape(B, heads, -1, d)
    kf = np.asarray(k, dtype=np.float64).reshape(B, heads, -1, d)
    vf = np.asarray(v, dtype=np.float64).reshape(B, heads, -1, d)
    out = np.empty(qf.shape, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            s = scale * (qf[b, h] @ kf[b, h].T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[b, h] = (p @ vf[b, h]) / p.sum(axis=1, keepdims=True)
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# Token order
# ----------------------------------------------------------------------------

def to_tile_major(x: np.ndarray, tile: Sequence[int]) -> np.ndarray:
    """(B, heads, T, H, W, d) raster -> (B, heads, n_tiles * tau, d) tile-major.

    Tiles in raster order of tile coordinates, tokens within a tile in raster
    order of their local coordinates; padded positions are zero rows.
    """
    B, heads, T, H, W, d = x.shape
    ct, ch, cw = tile
    nt, nh, nw = tile_grid((T, H, W), tile)
    xp = np.zeros((B, heads, nt * ct, nh * ch, nw * cw, d), dtype=x.dtype)
    xp[:, :, :T, :H, :W] = x
    y = xp.reshape(B, heads, nt, ct, nh, ch, nw, cw, d)
    y = y.transpose(0, 1, 2, 4, 6, 3, 5, 7, 8)
    return np.ascontiguousarray(y).reshape(B, heads, nt * nh * nw * ct * ch * cw, d)


def from_tile_major(y: np.ndarray, volume: Sequence[int], tile: Sequence[int]) -> np.ndarray:
    """Inverse of :func:`to_tile_major`: (B, heads, n_tiles * tau, d) ->
    (B, heads, T, H, W, d); padded rows are dropped."""
    B, heads, S, d = y.shape
    T, H, W = volume
    ct, ch, cw = tile
    nt, nh, nw = tile_grid(volume, tile)
    z = y.reshape(B, heads, nt, nh, nw, ct, ch, cw, d)
    z = z.transpose(0, 1, 2, 5, 3, 6, 4, 7, 8)
    z = z.reshape(B, heads, nt * ct, nh * ch, nw * cw, d)[:, :, :T, :H, :W]
    return np.ascontiguousarray(z)
