"""GPU: volumes the tile does not divide (tile grid padded up to whole tiles;
padding positions are neither keys nor outputs), against the float64 oracle:
the padded tile-major layout, tile lists, forward in both token orders, the
log-sum-exp, the backward and the window recall."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import (LSE_BF16_MAX_ABS, LSE_F32_MAX_ABS, RECALL_MAX_ABS, assert_close,
                               assert_grad_close, default_scale, e4m3_codes, e4m3_descale, to_gpu)

pytestmark = pytest.mark.gpu

CASES = [
    # name, volume, tile, windows per head, head_dim, dtype
    ("tile32_d64", (5, 6, 7), (2, 4, 4), [(4, 4, 4), (2, 8, 8), (6, 8, 8)], 64, "bf16"),
    ("tile96_d128", (7, 12, 20), (3, 4, 8), [(6, 8, 16), (9, 12, 24)], 128, "bf16"),
    ("tile384_hunyuan_like", (10, 20, 30), (6, 8, 8), [(6, 16, 16), (12, 24, 24)], 128, "bf16"),
    # tau = 192 and 384 with partly padded tiles: work items that start inside
    # a tile (rows 128.. and 256..) and may hold only padding rows
    ("tile192_items", (11, 9, 13), (4, 4, 12), [(8, 8, 12), (12, 12, 24)], 128, "bf16"),
    ("tile384_items", (13, 17, 19), (6, 8, 8), [(18, 24, 24)], 128, "bf16"),
]
# float32 attention on a padded grid is refused (STA_ERR_UNSUPPORTED): a first
# run of its padded forward faulted the GPU and the cause was not found, so
# that path was taken out; the float32 layout (reorder / restore) is kept.
F32_CASE = ("f32_tile32", (5, 6, 7), (2, 4, 4), [(4, 4, 4), (6, 8, 8)], 64, "f32")


def make(case, B=1, seed=41):
    name, volume, tile, windows, d, dtype = case
    w = workloads.small_case(volume, tile, windows, head_dim=d, dtype=dtype, B=B, seed=seed, name=name)
    return w, workloads.make_inputs(w)


@pytest.mark.parametrize("case", CASES + [F32_CASE], ids=lambda c: c[0])
def test_padded_layout_round_trip(case):
    w, inp = make(case, B=2)
    print(f"[case] padded layout {w}", flush=True)
    x = to_gpu(inp.q, w.dtype)
    tm = binding.sta_reorder_tiles(x, w.tile)
    assert tm.shape[2] == binding.tile_major_rows(w.volume, w.tile)
    ref = oracle.to_tile_major(inp.q, w.tile)
    assert np.array_equal(tm.float().cpu().numpy(), ref)   # padding rows are zero
    back = binding.sta_restore_order(tm, w.volume, w.tile)
    torch.cuda.synchronize()
    assert torch.equal(back, x)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_padded_tile_lists(case):
    _, volume, tile, windows, _, _ = case
    print(f"[case] padded tile lists {volume} {tile}", flush=True)
    kl, kc = binding.sta_kv_tiles(len(windows), volume, tile, windows)
    rl, rc = oracle.kv_tile_lists(volume, tile, np.array(windows), max_kv=kl.shape[-1])
    assert np.array_equal(kc.cpu().numpy(), rc) and np.array_equal(kl.cpu().numpy(), rl)
    ql, qc = binding.sta_q_tiles(len(windows), volume, tile, windows)
    rl, rc = oracle.q_tile_lists(volume, tile, windows, max_q=ql.shape[-1])
    assert np.array_equal(qc.cpu().numpy(), rc) and np.array_equal(ql.cpu().numpy(), rl)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_padded_forward_both_orders(case):
    w, inp = make(case, B=2)
    print(f"[case] padded forward {w}", flush=True)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    scale = default_scale(w.head_dim)
    fused = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, scale, fused=True)
    three = binding.sliding_tile_attention(q, k, v, w.tile, inp.windows, scale, fused=False)
    torch.cuda.synchronize()
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, scale)
    assert_close(fused.float().cpu().numpy(), ref, w.dtype, f"{w.name} raster")
    assert torch.equal(fused, three)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_padded_lse(case):
    w, inp = make(case)
    print(f"[case] padded lse {w}", flush=True)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    _, lse = binding.sta_forward_lse(q, k, v, w.tile, inp.windows)
    torch.cuda.synchronize()
    ref = oracle.sta_lse(inp.q, inp.k, w.tile, inp.windows, default_scale(w.head_dim))
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref).max()
    print(f"[parity] {w.name} lse max_abs {err:.3e}", flush=True)
    assert err <= (LSE_BF16_MAX_ABS if w.dtype == "bf16" else LSE_F32_MAX_ABS)


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_padded_backward(case, order):
    w, inp = make(case, B=2, seed=42)
    print(f"[case] padded backward {order} {w}", flush=True)
    dout = workloads.make_grad_output(w)
    q, k, v, do = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v, dout))
    scale = default_scale(w.head_dim)
    if order == "raster":
        out, lse = binding.sta_forward_lse(q, k, v, w.tile, inp.windows, scale)
        grads = binding.sta_backward(q, k, v, out, do, lse, w.tile, inp.windows, scale)
    else:
        qt, kt, vt, dot = (binding.sta_reorder_tiles(x, w.tile) for x in (q, k, v, do))
        out, lse = binding.sta_forward_lse(qt, kt, vt, w.tile, inp.windows, scale, volume=w.volume)
        g = binding.sta_backward(qt, kt, vt, out, dot, lse, w.tile, inp.windows, scale, volume=w.volume)
        grads = [binding.sta_restore_order(x, w.volume, w.tile) for x in g]
    torch.cuda.synchronize()
    ref = oracle.sta_backward(inp.q, inp.k, inp.v, dout, w.tile, inp.windows, scale)
    for nm, g, r in zip(("dq", "dk", "dv"), grads, ref):
        assert_grad_close(g.float().cpu().numpy(), r, w.dtype, f"{w.name} {order} {nm}")


def test_padded_float32_attention_is_refused():
    """Refused before any launch (argument check on the host)."""
    w, inp = make(F32_CASE)
    q, k, v = (to_gpu(x, "f32") for x in (inp.q, inp.k, inp.v))
    with pytest.raises(NotImplementedError, match="float32"):
        binding.sta_forward_raster(q, k, v, w.tile, inp.windows)
    with pytest.raises(NotImplementedError, match="float32"):
        binding.sta_forward_lse(q, k, v, w.tile, inp.windows)
    with pytest.raises(NotImplementedError, match="float32"):
        binding.sta_window_recall(q, k, w.tile, [(4, 4, 4)])
    qt = binding.sta_reorder_tiles(q, w.tile)
    with pytest.raises(NotImplementedError, match="float32"):
        binding.sta_forward(qt, qt.clone(), qt.clone(), w.volume, w.tile, inp.windows)
    lse = torch.zeros(q.shape[:-1], dtype=torch.float32, device="cuda")
    with pytest.raises(NotImplementedError, match="float32"):
        binding.sta_backward(q, k, v, q.clone(), q.clone(), lse, w.tile, inp.windows)


def test_padded_recall_raster_and_tile_major_refused():
    w, inp = make(CASES[1])
    print(f"[case] padded recall {w}", flush=True)
    q, k = to_gpu(inp.q, "bf16"), to_gpu(inp.k, "bf16")
    cands = [(3, 4, 8), (6, 8, 16), (9, 12, 24)]
    got = binding.sta_window_recall(q, k, w.tile, cands)
    torch.cuda.synchronize()
    ref = oracle.window_recall(inp.q, inp.k, w.tile, cands, default_scale(w.head_dim))
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
    print(f"[parity] padded recall max_abs {err:.3e}", flush=True)
    assert err <= RECALL_MAX_ABS
    qt, kt = binding.sta_reorder_tiles(q, w.tile), binding.sta_reorder_tiles(k, w.tile)
    with pytest.raises(NotImplementedError):
        binding.sta_window_recall(qt, kt, w.tile, cands, volume=w.volume)


def _poison_padding_rows(x_tm: torch.Tensor, real: torch.Tensor) -> torch.Tensor:
    """A tile-major tensor whose padding rows hold NaN (real: bool (S_pad,))."""
    y = x_tm.clone()
    y[:, :, ~real] = float("nan")
    return y


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=lambda c: c[0])
def test_padded_tile_major_ignores_padding_row_contents(case):
    """Tile-major tensors of a padded grid: whatever a caller keeps in the
    padding rows (here NaN in q, k, v, out and dout) never reaches the real
    outputs: forward, lse, fp8 forward and the gradients equal the oracle."""
    w, inp = make(case, B=2, seed=43)
    print(f"[case] padded tile-major NaN padding rows {w}", flush=True)
    scale = default_scale(w.head_dim)
    q, k, v = (to_gpu(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    ones = torch.ones_like(q[:1, :1])
    real = binding.sta_reorder_tiles(ones, w.tile)[0, 0, :, 0] != 0   # padding rows are zeros
    assert not bool(real.all())
    qt, kt, vt = (_poison_padding_rows(binding.sta_reorder_tiles(x, w.tile), real) for x in (q, k, v))
    out, lse = binding.sta_forward_lse(qt, kt, vt, w.tile, inp.windows, scale, volume=w.volume)
    torch.cuda.synchronize()
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, scale)
    got = binding.sta_restore_order(out, w.volume, w.tile)
    assert_close(got.float().cpu().numpy(), ref, w.dtype, f"{w.name} tile-major NaN padding")
    ref_lse = oracle.to_tile_major(oracle.sta_lse(inp.q, inp.k, w.tile, inp.windows, scale)[..., None],
                                   w.tile)[..., 0]
    lerr = np.abs(lse.cpu().numpy()[:, :, real.cpu().numpy()] - ref_lse[:, :, real.cpu().numpy()]).max()
    print(f"[parity] {w.name} tile-major NaN padding lse max_abs {lerr:.3e}", flush=True)
    assert lerr <= LSE_BF16_MAX_ABS
    # fp8 q and k (0x7F is a NaN code) with NaN V padding rows
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    q8t, k8t = (torch.from_numpy(oracle.to_tile_major(x, w.tile)).cuda() for x in (q8, k8))
    if w.head_dim == 128:
        for x in (q8t, k8t):
            x[:, :, ~real] = 0x7F
        o8 = binding.sta_forward_fp8(q8t, k8t, vt, w.tile, inp.windows, qd, kd, scale, volume=w.volume)
        torch.cuda.synchronize()
        ref8 = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, scale, qd, kd)
        assert_close(binding.sta_restore_order(o8, w.volume, w.tile).float().cpu().numpy(), ref8, "bf16",
                     f"{w.name} fp8 tile-major NaN padding")
    # backward with NaN padding rows in out and dout as well
    dout = workloads.make_grad_output(w)
    dot = _poison_padding_rows(binding.sta_reorder_tiles(to_gpu(dout, w.dtype), w.tile), real)
    out = _poison_padding_rows(out, real)
    g = binding.sta_backward(qt, kt, vt, out, dot, lse, w.tile, inp.windows, scale, volume=w.volume)
    grads = [binding.sta_restore_order(x, w.volume, w.tile) for x in g]
    torch.cuda.synchronize()
    gref = oracle.sta_backward(inp.q, inp.k, inp.v, dout, w.tile, inp.windows, scale)
    for nm, a, r in zip(("dq", "dk", "dv"), grads, gref):
        assert_grad_close(a.float().cpu().numpy(), r, w.dtype, f"{w.name} tile-major NaN padding {nm}")
