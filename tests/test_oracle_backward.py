"""Pins for the backward and log-sum-exp parts of the CPU oracle.

None of these tests calls the HIP library. Each compares the oracle with
something other than itself: central finite differences of the (separately
pinned) forward oracle, torch autograd through a library softmax attention,
a library log-sum-exp, brute-force transposed tile lists, and invariants of
softmax attention that hold for any mask.
"""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

TINY = dict(volume=(4, 4, 6), tile=(2, 2, 2))


def draw(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(4)]


def loss(q, k, v, dout, tile, windows, scale):
    return float(np.sum(dout * oracle.sta_attention(q, k, v, tile, windows, scale)))


@pytest.mark.parametrize("windows", [[(2, 2, 4), (4, 4, 6)], [(2, 4, 2), (4, 2, 4)]])
def test_gradients_match_central_differences(windows):
    """dq, dk, dv equal the central differences of sum(dout * O) taken on the
    forward oracle, at 40 random coordinates of each tensor."""
    vol, tile = TINY["volume"], TINY["tile"]
    shape = (1, len(windows)) + vol + (8,)
    q, k, v, dout = draw(shape, 7)
    scale = 0.4
    dq, dk, dv = oracle.sta_backward(q, k, v, dout, tile, windows, scale)
    rng = np.random.default_rng(1)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(40):
            idx = tuple(int(rng.integers(0, s)) for s in shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], dout, tile, windows, scale)
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], dout, tile, windows, scale)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 + 1e-6 * abs(fd), (name, idx, fd, g[idx])


def _autograd_sdpa(q, k, v, dout, scale):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_whole_volume_window_equals_library_attention_gradient():
    vol, tile = (4, 4, 6), (2, 2, 2)
    shape = (2, 2) + vol + (8,)
    q, k, v, dout = draw(shape, 8)
    scale = 0.35
    got = oracle.sta_backward(q, k, v, dout, tile, [vol, vol], scale)
    flat = lambda a: a.reshape(2, 2, -1, 8)  # noqa: E731
    ref = _autograd_sdpa(flat(q), flat(k), flat(v), flat(dout), scale)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(flat(g), r, rtol=1e-10, atol=1e-12)


def test_single_tile_window_is_per_tile_attention_gradient():
    """A window of one tile makes attention block-diagonal over tiles: the
    gradient is that of independent attention inside every tile."""
    vol, tile = (4, 4, 6), (2, 2, 2)
    shape = (1, 1) + vol + (8,)
    q, k, v, dout = draw(shape, 9)
    scale = 0.5
    dq, dk, dv = oracle.sta_backward(q, k, v, dout, tile, [tile], scale)
    tm = lambda a: oracle.to_tile_major(a, tile).reshape(1, 1, -1, 8, 8)  # noqa: E731
    ref = _autograd_sdpa(tm(q), tm(k), tm(v), tm(dout), scale)  # batched over tiles
    for g, r in zip((dq, dk, dv), ref):
        np.testing.assert_allclose(tm(g), r, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("window", [(2, 2, 2), (2, 4, 4), (4, 2, 6)])
def test_gradient_invariants(window):
    """Shifting every key by one vector leaves each row's softmax unchanged, so
    the dK rows sum to zero; adding one vector to every value adds it to every
    output, so the dV rows sum to the dO rows' sum; and scores are bilinear in
    q and k, so sum(dq * q) = sum(dk * k)."""
    vol, tile = TINY["volume"], TINY["tile"]
    shape = (1, 1) + vol + (8,)
    q, k, v, dout = draw(shape, 10)
    dq, dk, dv = oracle.sta_backward(q, k, v, dout, tile, [window], 0.6)
    np.testing.assert_allclose(dk.reshape(-1, 8).sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.reshape(-1, 8).sum(axis=0), dout.reshape(-1, 8).sum(axis=0), atol=1e-12)
    assert abs(np.sum(dq * q) - np.sum(dk * k)) <= 1e-11


def test_row_subsets_match_full_backward():
    """The row-subset gradients (used by the sampled full-size checks) equal
    the matching rows of the whole backward for every (b, h) of a B = 2,
    two-head draw with a different window per head."""
    vol, tile = (6, 4, 6), (2, 2, 2)
    windows = [(4, 2, 4), (2, 4, 6)]
    shape = (2, 2) + vol + (8,)
    q, k, v, dout = draw(shape, 11)
    dq, dk, dv = oracle.sta_backward(q, k, v, dout, tile, windows, 0.3)
    rows = np.array([0, 5, 17, 40, 77, 143])
    for b in range(2):
        for h in range(2):
            gq = oracle.sta_backward_query_rows(q, k, v, dout, tile, windows[h], 0.3, b, h, rows)
            gk, gv = oracle.sta_backward_key_rows(q, k, v, dout, tile, windows[h], 0.3, b, h, rows)
            np.testing.assert_allclose(gq, dq[b, h].reshape(-1, 8)[rows], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(gk, dk[b, h].reshape(-1, 8)[rows], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(gv, dv[b, h].reshape(-1, 8)[rows], rtol=1e-12, atol=1e-13)


def test_lse_whole_volume_is_library_logsumexp():
    vol, tile = (4, 4, 6), (2, 2, 2)
    q, k, _, _ = draw((1, 2) + vol + (8,), 12)
    got = oracle.sta_lse(q, k, tile, [vol, vol], 0.4)
    for h in range(2):
        s = 0.4 * q[0, h].reshape(-1, 8) @ k[0, h].reshape(-1, 8).T
        np.testing.assert_allclose(got[0, h].reshape(-1), logsumexp(s, axis=1), rtol=1e-13)


def test_lse_of_zero_query_is_log_of_window_size():
    vol, tile, window = (6, 4, 6), (2, 2, 2), (4, 2, 4)
    _, k, _, _ = draw((1, 1) + vol + (8,), 13)
    q = np.zeros((1, 1) + vol + (8,))
    got = oracle.sta_lse(q, k, tile, [window], 1.0)
    np.testing.assert_allclose(got, np.log(4 * 2 * 4), rtol=1e-14)


@pytest.mark.parametrize("volume,tile,window", [
    ((10, 4, 10), (1, 1, 1), (3, 1, 3)),
    ((10, 12, 6), (2, 2, 2), (6, 4, 6)),
    ((8, 8, 8), (2, 2, 2), (4, 8, 2)),
    ((30, 48, 80), (6, 8, 8), (18, 24, 24)),
])
def test_query_tile_lists_are_the_transposed_window(volume, tile, window):
    """Key tile j lists query tile i iff i's window holds j (brute force over
    the per-axis clamped windows); counts total N_t * prod(omega); per axis the
    query tiles of a key tile form one contiguous interval."""
    n = oracle.tile_grid(volume, tile)
    om = [w // c for w, c in zip(window, tile)]
    lists, counts = oracle.q_tile_lists(volume, tile, [window])
    n_tiles = n[0] * n[1] * n[2]
    assert counts.sum() == n_tiles * om[0] * om[1] * om[2]
    coords = [(t, y, x) for t in range(n[0]) for y in range(n[1]) for x in range(n[2])]
    for j, kc in enumerate(coords):
        want = []
        for i, qc in enumerate(coords):
            st = [oracle.window_start(qc[a], n[a], om[a]) for a in range(3)]
            if all(st[a] <= kc[a] < st[a] + om[a] for a in range(3)):
                want.append(i)
        assert list(lists[0, j, : counts[0, j]]) == want
        per_axis = [sorted({coords[i][a] for i in want}) for a in range(3)]
        for a in range(3):
            assert per_axis[a] == list(range(per_axis[a][0], per_axis[a][-1] + 1))


def test_transposed_window_is_not_symmetric_under_clamping():
    """At the pages' 30x48x80 / (6,8,8) / (18,24,24) the corner key tile is seen
    by 2 x 2 x 2 query tiles and a centre one by 3 x 3 x 3, although every query
    tile sees 27 key tiles."""
    _, counts = oracle.q_tile_lists((30, 48, 80), (6, 8, 8), [(18, 24, 24)])
    assert counts[0, 0] == 8
    assert counts.min() == 8 and counts.max() > 27
    assert counts.sum() == 300 * 27


# ----------------------------------------------------------------------------
# Window recall
# ----------------------------------------------------------------------------

RECALL_VOL, RECALL_TILE = (6, 4, 6), (2, 2, 2)
RECALL_CANDS = [(2, 2, 2), (4, 2, 4), (2, 4, 6), (6, 4, 6)]


def test_recall_equals_lse_difference_from_a_library_logsumexp():
    """recall = mean_i exp(lse_window(i) - logsumexp over all keys(i)); the full
    log-sum-exp here comes from scipy, the window one from the pinned lse."""
    q, k, _, _ = draw((2, 2) + RECALL_VOL + (8,), 14)
    got = oracle.window_recall(q, k, RECALL_TILE, RECALL_CANDS, 0.5)
    for b in range(2):
        for h in range(2):
            s = 0.5 * q[b, h].reshape(-1, 8) @ k[b, h].reshape(-1, 8).T
            full = logsumexp(s, axis=1)
            for c, w in enumerate(RECALL_CANDS):
                lw = oracle.sta_lse(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], RECALL_TILE, [w], 0.5)
                want = np.mean(np.exp(lw.reshape(-1) - full))
                assert abs(got[b, h, c] - want) <= 1e-12


def test_recall_special_cases():
    """Whole-volume window keeps everything; with q = 0 attention is uniform, so
    a window keeps its share of the keys; recall grows with nested windows."""
    q, k, _, _ = draw((1, 1) + RECALL_VOL + (8,), 15)
    got = oracle.window_recall(q, k, RECALL_TILE, RECALL_CANDS, 0.7)[0, 0]
    assert abs(got[-1] - 1.0) <= 1e-12
    assert 0 < got[0] < got[1] < got[-1]   # (2,2,2) inside (4,2,4) inside the volume
    S = 6 * 4 * 6
    zero = oracle.window_recall(np.zeros_like(q), k, RECALL_TILE, RECALL_CANDS, 0.7)[0, 0]
    for c, w in enumerate(RECALL_CANDS):
        assert abs(zero[c] - w[0] * w[1] * w[2] / S) <= 1e-12
