"""GPU: forward log-sum-exp, transposed tile lists and the STA backward
(dq, dk, dv) against the float64 oracle, in both token orders, on small
seeded workloads that span several tiles (with ragged key chunks), and on
sampled rows at the 30x48x80 headline shape."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import (LSE_BF16_MAX_ABS, LSE_F32_MAX_ABS, assert_grad_close, default_scale,
                               to_gpu)

pytestmark = pytest.mark.gpu

CASES = [
    # name, volume, tile, windows per head, head_dim, dtype
    ("tiles_6x8x8_two_heads", (12, 16, 24), (6, 8, 8), [(6, 8, 8), (12, 16, 24)], 128, "bf16"),
    ("tile64_w333_and_even", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (8, 8, 8)], 128, "bf16"),
    ("tile64_d64", (12, 16, 16), (4, 4, 4), [(4, 8, 12)], 64, "bf16"),
    ("tile48_ragged", (9, 8, 12), (3, 4, 4), [(6, 4, 8), (9, 8, 12)], 128, "bf16"),
    ("tile128", (8, 8, 16), (4, 4, 8), [(4, 8, 8)], 128, "bf16"),
    ("tile192", (9, 16, 24), (3, 8, 8), [(6, 16, 16), (9, 8, 24)], 128, "bf16"),
    ("tile8_tiny", (4, 4, 6), (2, 2, 2), [(2, 2, 2), (4, 2, 4)], 64, "bf16"),
    ("image_2d_tile8x8", (1, 32, 48), (1, 8, 8), [(1, 24, 24), (1, 8, 16)], 128, "bf16"),
    ("f32_d64", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 8, 12)], 64, "f32"),
    ("f32_d128_ragged", (9, 8, 12), (3, 4, 4), [(6, 4, 8)], 128, "f32"),
]


def gpu(inp, dout=None):
    w = inp.workload
    ts = [to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v)]
    if dout is not None:
        ts.append(to_gpu(dout, w.dtype))
    return ts


def tm(x, tile):
    """Raster (B, heads, T, H, W, d) tensor -> tile-major (B, heads, S, d) via the library."""
    return binding.sta_reorder_tiles(x, tile)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_q_tiles_bit_exact(case):
    _, volume, tile, windows, _, _ = case
    print(f"[case] q_tiles {volume} {tile} {windows}", flush=True)
    lists, counts = binding.sta_q_tiles(len(windows), volume, tile, windows)
    ref_l, ref_c = oracle.q_tile_lists(volume, tile, windows, max_q=lists.shape[-1])
    assert np.array_equal(counts.cpu().numpy(), ref_c)
    assert np.array_equal(lists.cpu().numpy(), ref_l)


def test_q_tiles_headline_geometry():
    win = [(18, 24, 24), (30, 40, 40), (30, 48, 80)]
    lists, counts = binding.sta_q_tiles(3, (30, 48, 80), (6, 8, 8), win)
    ref_l, ref_c = oracle.q_tile_lists((30, 48, 80), (6, 8, 8), win, max_q=lists.shape[-1])
    assert np.array_equal(counts.cpu().numpy(), ref_c)
    assert np.array_equal(lists.cpu().numpy(), ref_l)


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_forward_lse(case, order):
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, B=2, seed=21, name=name)
    print(f"[case] forward_lse {order} {w}", flush=True)
    inp = workloads.make_inputs(w)
    q, k, v = gpu(inp)
    scale = default_scale(d)
    if order == "raster":
        out, lse = binding.sta_forward_lse(q, k, v, tile, inp.windows, scale)
        plain = binding.sta_forward_raster(q, k, v, tile, inp.windows, scale)
        lse_r = lse
    else:
        qt, kt, vt = (tm(x, tile) for x in (q, k, v))
        out, lse = binding.sta_forward_lse(qt, kt, vt, tile, inp.windows, scale, volume=volume)
        plain = binding.sta_forward(qt, kt, vt, volume, tile, inp.windows, scale)
        # tile-major lse rows -> raster via the library permutation of a 16-byte-row view
        lse_r = binding.sta_restore_order(lse.unsqueeze(-1).expand(*lse.shape, 4).contiguous(),
                                          volume, tile)[..., 0]
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "output differs from the forward without lse"
    ref = oracle.sta_lse(inp.q, inp.k, tile, inp.windows, scale)
    err = np.abs(lse_r.cpu().numpy().astype(np.float64) - ref).max()
    print(f"[parity] {name} lse max_abs {err:.3e}", flush=True)
    assert err <= (LSE_BF16_MAX_ABS if dtype == "bf16" else LSE_F32_MAX_ABS)


def run_backward(inp, dout, order, scale):
    w = inp.workload
    q, k, v, do = gpu(inp, dout)
    if order == "raster":
        out, lse = binding.sta_forward_lse(q, k, v, w.tile, inp.windows, scale)
        grads = binding.sta_backward(q, k, v, out, do, lse, w.tile, inp.windows, scale)
    else:
        qt, kt, vt, dot = (tm(x, w.tile) for x in (q, k, v, do))
        out, lse = binding.sta_forward_lse(qt, kt, vt, w.tile, inp.windows, scale, volume=w.volume)
        g = binding.sta_backward(qt, kt, vt, out, dot, lse, w.tile, inp.windows, scale, volume=w.volume)
        grads = tuple(binding.sta_restore_order(x, w.volume, w.tile) for x in g)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_backward_matches_oracle(case, order):
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, B=2, seed=22, name=name)
    print(f"[case] backward {order} {w}", flush=True)
    inp = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w)
    scale = default_scale(d)
    got = run_backward(inp, dout, order, scale)
    ref = oracle.sta_backward(inp.q, inp.k, inp.v, dout, tile, inp.windows, scale)
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert_grad_close(g.float().cpu().numpy(), r, dtype, f"{name} {order} {nm}")


@pytest.mark.parametrize("case", [c for c in CASES if c[0] not in ("tile128", "tile8_tiny")],
                         ids=lambda c: c[0])
def test_backward_orders_agree_bit_for_bit(case):
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, seed=23, name=name)
    print(f"[case] backward raster vs tile-major {w}", flush=True)
    inp = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w)
    a = run_backward(inp, dout, "raster", 0.1)
    b = run_backward(inp, dout, "tile_major", 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_is_deterministic():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 16, 8)], seed=24, name="det")
    print(f"[case] backward determinism {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w)
    a = run_backward(inp, dout, "raster", 0.09)
    b = run_backward(inp, dout, "raster", 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_matches_entry_points():
    w = workloads.small_case((12, 16, 16), (4, 4, 4), [(8, 8, 8), (12, 12, 12)], seed=25, name="autograd")
    print(f"[case] autograd {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w)
    q, k, v, do = gpu(inp, dout)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = binding.sta_attention(qa, ka, va, w.tile, inp.windows)
    out.backward(do)
    ref_out, lse = binding.sta_forward_lse(q, k, v, w.tile, inp.windows)
    dq, dk, dv = binding.sta_backward(q, k, v, ref_out, do, lse, w.tile, inp.windows)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


def test_zero_upstream_gradient_gives_zero():
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 8, 8)], seed=26, name="zero_dout")
    print(f"[case] backward {w.name}", flush=True)
    inp = workloads.make_inputs(w)
    dout = np.zeros_like(inp.q)
    for g in run_backward(inp, dout, "raster", 0.1):
        assert torch.count_nonzero(g).item() == 0


def sample_tokens(volume, tile, rng, tiles):
    out = []
    for t in tiles:
        toks = oracle.tile_tokens(volume, tile, t)
        out.append(np.unique(np.concatenate([toks[[0, -1]], rng.choice(toks, 4, replace=False)])))
    return np.concatenate(out)


@pytest.mark.timeout(400)   # input draws, the backward, then the oracle's rows on the host
@pytest.mark.parametrize("wl", [workloads.STA_18_24_24, workloads.MIXED_HEADS], ids=lambda w: w.name)
def test_backward_full_size_sampled_rows(wl):
    """At 30x48x80 (24 heads, d=128, bf16), in the raster launch configuration:
    dq on sampled query rows of corner, edge and interior tiles, and dk, dv on
    sampled key rows of a corner and an interior tile, against the oracle row
    by row. (The oracle's key-row gradient needs every query tile that reads
    the key tile, over all S keys each, so key rows are sampled from two heads
    whose window is not the whole volume.)"""
    print(f"[case] backward full size {wl.name}: inputs", flush=True)
    inp = workloads.make_inputs(wl)
    dout = workloads.make_grad_output(wl)
    scale = default_scale(wl.head_dim)
    print(f"[case] backward full size {wl.name}: running", flush=True)
    dq, dk, dv = run_backward(inp, dout, "raster", scale)
    flat = lambda x: x.float().cpu().numpy().reshape(wl.B, wl.heads, -1, wl.head_dim)  # noqa: E731
    dq, dk, dv = flat(dq), flat(dk), flat(dv)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    rng = np.random.default_rng(wl.seed)
    n = oracle.tile_grid(wl.volume, wl.tile)
    n_tiles = n[0] * n[1] * n[2]
    interior = ((n[0] // 2) * n[1] + n[1] // 2) * n[2] + n[2] // 2
    edge = (n[1] - 1) * n[2] + n[2] // 2
    whole = tuple(wl.volume)
    heads = sorted({0, wl.heads - 1, int(rng.integers(0, wl.heads))})
    key_heads = [h for h in range(wl.heads) if tuple(inp.windows[h]) != whole][:1] + \
        [h for h in reversed(range(wl.heads)) if tuple(inp.windows[h]) != whole][:1]
    for h in heads:
        window = tuple(int(x) for x in inp.windows[h])
        rows = sample_tokens(wl.volume, wl.tile, rng, [0, n_tiles - 1, interior, edge])
        gq = oracle.sta_backward_query_rows(inp.q, inp.k, inp.v, dout, wl.tile, window, scale, 0, h, rows)
        assert_grad_close(dq[0, h, rows], gq, "bf16", f"{wl.name} head {h} {window} dq")
    if wl is workloads.STA_18_24_24:
        # every row of the last four query tiles of every head (the query
        # side's work items of each XCD's last, partly filled round)
        rows = np.concatenate([oracle.tile_tokens(wl.volume, wl.tile, t) for t in range(n_tiles - 4, n_tiles)])
        print(f"[case] backward full size {wl.name}: dq of the last four tiles of every head", flush=True)
        for h in range(wl.heads):
            window = tuple(int(x) for x in inp.windows[h])
            gq = oracle.sta_backward_query_rows(inp.q, inp.k, inp.v, dout, wl.tile, window, scale, 0, h, rows)
            assert_grad_close(dq[0, h, rows], gq, "bf16", f"{wl.name} head {h} dq, last tiles")
    for h in sorted(set(key_heads)):
        window = tuple(int(x) for x in inp.windows[h])
        rows = sample_tokens(wl.volume, wl.tile, rng, [0, interior])
        print(f"[case] oracle key rows head {h} {window}", flush=True)
        gk, gv = oracle.sta_backward_key_rows(inp.q, inp.k, inp.v, dout, wl.tile, window, scale, 0, h, rows)
        assert_grad_close(dk[0, h, rows], gk, "bf16", f"{wl.name} head {h} {window} dk")
        assert_grad_close(dv[0, h, rows], gv, "bf16", f"{wl.name} head {h} {window} dv")
