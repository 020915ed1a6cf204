"""CPU oracle for the STA backward pass and the log-sum-exp of the forward --
TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module. It shares no code with the HIP library and never calls it.

The pages train the model with a fixed STA window (atlas.scime.ai summary,
"Approach" and "Experimental setup", fine-tuning with attention distillation;
podcast transcript, the answer on fine-tuning), which needs the gradient of the
STA output with respect to q, k and v. STA is masked softmax attention with a
tile-structured mask, so the gradient is the plain gradient of
    O = P V,  P = softmax_row(scale * Q K^T restricted to the visible keys):
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),  D_i = sum_j P_ij dP_ij = dO_i . O_i
    dQ = scale * dS K
    dK = scale * dS^T Q
with P = 0 (hence dS = 0) on keys the query does not see. The log-sum-exp of a
query row is lse_i = log sum_j exp(scale * q_i . k_j) over its visible keys, so
P_ij = exp(scale * q_i . k_j - lse_i).

The visible keys of a query are those of :mod:`sta_oracle` (token mask from
token coordinates, clamped window). The query tiles that see a key tile are the
transpose of the tile selection; under the clamped window this is not the same
as the key tiles a query tile sees.

All arithmetic is float64. Query rows are processed one tile at a time.
"""

from __future__ import annotations

import numpy as np

from .sta_oracle import tile_grid, tile_selection, tile_tokens, token_mask_rows


def _rows_f64(x, b, h):
    d = x.shape[-1]
    return np.asarray(x[b, h], dtype=np.float64).reshape(-1, d)


def _softmax_rows(q_rows, k_all, allowed, scale):
    """P (masked rows, float64) and lse of each row (natural log)."""
    s = scale * (q_rows @ k_all.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise AssertionError("a query row sees no key")
    e = np.where(allowed, np.exp(s - m), 0.0)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def sta_lse(q, k, tile, windows, scale) -> np.ndarray:
    """Log-sum-exp of every query row over its visible keys, float64, shape
    (B, heads, T, H, W), raster order."""
    B, heads = q.shape[:2]
    volume = q.shape[2:5]
    windows = np.asarray(windows).reshape(heads, 3)
    n = tile_grid(volume, tile)
    out = np.empty(q.shape[:5], dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            qf, kf = _rows_f64(q, b, h), _rows_f64(k, b, h)
            of = out[b, h].reshape(-1)
            w = tuple(int(x) for x in windows[h])
            for i in range(n[0] * n[1] * n[2]):
                rows = tile_tokens(volume, tile, i)
                _, lse = _softmax_rows(qf[rows], kf, token_mask_rows(volume, tile, w, rows), scale)
                of[rows] = lse
    return out


def q_tile_lists(volume, tile, windows, max_q: int | None = None):
    """Per head and key tile: the query tiles whose window holds it, ascending.

    Returns (lists int32 [heads, N_t, max_q] padded with -1, counts int32 [heads, N_t]).
    """
    windows = np.asarray(windows).reshape(-1, 3)
    sels = [tile_selection(volume, tile, tuple(int(x) for x in w)).T for w in windows]
    n_tiles = sels[0].shape[0]
    counts = np.stack([s.sum(axis=1) for s in sels]).astype(np.int32)
    if max_q is None:
        max_q = int(counts.max())
    lists = np.full((len(sels), n_tiles, max_q), -1, dtype=np.int32)
    for h, s in enumerate(sels):
        for j in range(n_tiles):
            idx = np.nonzero(s[j])[0]
            lists[h, j, : len(idx)] = idx
    return lists, counts


def _tile_backward(qf, kf, vf, dof, rows, allowed, scale):
    """Gradient contributions of the query rows ``rows`` (one tile).

    Returns dQ rows and the (S, d) contributions to dK and dV.
    """
    p, _ = _softmax_rows(qf[rows], kf, allowed, scale)
    o = p @ vf
    do = dof[rows]
    dpr = do @ vf.T
    delta = np.sum(do * o, axis=1, keepdims=True)
    ds = p * (dpr - delta)
    return scale * (ds @ kf), scale * (ds.T @ qf[rows]), p.T @ do


def sta_backward(q, k, v, dout, tile, windows, scale):
    """Gradients (dq, dk, dv) of sum(dout * STA(q, k, v)), float64, each shaped
    like q (B, heads, T, H, W, d), raster order."""
    B, heads = q.shape[:2]
    volume = q.shape[2:5]
    d = q.shape[-1]
    windows = np.asarray(windows).reshape(heads, 3)
    n = tile_grid(volume, tile)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(q.shape, dtype=np.float64)
    dv = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            qf, kf, vf, dof = (_rows_f64(x, b, h) for x in (q, k, v, dout))
            dqf = dq[b, h].reshape(-1, d)
            dkf = dk[b, h].reshape(-1, d)
            dvf = dv[b, h].reshape(-1, d)
            w = tuple(int(x) for x in windows[h])
            for i in range(n[0] * n[1] * n[2]):
                rows = tile_tokens(volume, tile, i)
                allowed = token_mask_rows(volume, tile, w, rows)
                gq, gk, gv = _tile_backward(qf, kf, vf, dof, rows, allowed, scale)
                dqf[rows] = gq
                dkf += gk
                dvf += gv
    return dq, dk, dv


def _visible_columns(allowed):
    """Key tokens some query row of ``allowed`` sees; every other key has
    P = 0 for all these rows and drops out of every sum."""
    return np.nonzero(allowed.any(axis=0))[0]


def sta_backward_query_rows(q, k, v, dout, tile, window, scale, b, h, query_tokens):
    """dQ for the given raster query tokens of (b, h), float64 (R, d)."""
    volume = q.shape[2:5]
    qf, kf, vf, dof = (_rows_f64(x, b, h) for x in (q, k, v, dout))
    rows = np.asarray(query_tokens)
    allowed = token_mask_rows(volume, tile, window, rows)
    cols = _visible_columns(allowed)
    p, _ = _softmax_rows(qf[rows], kf[cols], allowed[:, cols], scale)
    o = p @ vf[cols]
    do = dof[rows]
    ds = p * (do @ vf[cols].T - np.sum(do * o, axis=1, keepdims=True))
    return scale * (ds @ kf[cols])


def sta_backward_key_rows(q, k, v, dout, tile, window, scale, b, h, key_tokens):
    """dK and dV for the given raster key tokens of (b, h), float64 (R, d) each.

    Every query tile whose window holds one of the keys' tiles contributes; its
    softmax is normalised over all of its visible keys.
    """
    volume = q.shape[2:5]
    n = tile_grid(volume, tile)
    qf, kf, vf, dof = (_rows_f64(x, b, h) for x in (q, k, v, dout))
    keys = np.asarray(key_tokens)
    sel = tile_selection(volume, tile, window)
    # tile index of each key token
    T, H, W = volume
    t, rem = np.divmod(keys, H * W)
    y, x = np.divmod(rem, W)
    kt = ((t // tile[0]) * n[1] + y // tile[1]) * n[2] + x // tile[2]
    q_tiles = np.nonzero(sel[:, np.unique(kt)].any(axis=1))[0]
    d = q.shape[-1]
    gk = np.zeros((len(keys), d))
    gv = np.zeros((len(keys), d))
    for i in q_tiles:
        rows = tile_tokens(volume, tile, int(i))
        allowed = token_mask_rows(volume, tile, window, rows)
        cols = _visible_columns(allowed)
        p, _ = _softmax_rows(qf[rows], kf[cols], allowed[:, cols], scale)
        o = p @ vf[cols]
        do = dof[rows]
        delta = np.sum(do * o, axis=1, keepdims=True)
        # P of the requested keys (0 where the tile does not see the key)
        pos = np.minimum(np.searchsorted(cols, keys), len(cols) - 1)
        pk = np.where((cols[pos] == keys)[None, :], p[:, pos], 0.0)
        ds = pk * (do @ vf[keys].T - delta)
        gk += scale * (ds.T @ qf[rows])
        gv += pk.T @ do
    return gk, gv


def window_recall(q, k, tile, candidates, scale) -> np.ndarray:
    """Attention recall, float64 (B, heads, n_candidates): for each candidate
    window, the mean over query rows of the full-attention probability (softmax
    over all keys) that falls on the keys the window shows the row (podcast
    transcript, the answer on attention recall; dianyo ICML2025 blog, STA
    section)."""
    B, heads = q.shape[:2]
    volume = q.shape[2:5]
    candidates = [tuple(int(x) for x in c) for c in np.asarray(candidates).reshape(-1, 3)]
    n = tile_grid(volume, tile)
    S = volume[0] * volume[1] * volume[2]
    out = np.zeros((B, heads, len(candidates)), dtype=np.float64)
    for b in range(B):
        for h in range(heads):
            qf, kf = _rows_f64(q, b, h), _rows_f64(k, b, h)
            for i in range(n[0] * n[1] * n[2]):
                rows = tile_tokens(volume, tile, i)
                p, _ = _softmax_rows(qf[rows], kf, np.ones((len(rows), S), dtype=bool), scale)
                for c, w in enumerate(candidates):
                    out[b, h, c] += np.sum(p[token_mask_rows(volume, tile, w, rows)])
    return out / S
