"""GPU: STA forward with fp8 (OCP E4M3) queries and keys against the float64
oracle on the same codes, in both token orders, on small seeded workloads
(several tiles, ragged runs, a padded tile grid, per-head windows) and on
sampled rows of the 30x48x80 workload in the launch configuration of the
raster-order kernel; plus agreement with the bf16 kernel on the decoded values
(every E4M3 value times a power-of-two descale is a bf16 value). The row
log-sum-exp of the fp8 scores, and the training path it enables (the bf16
backward on the decoded q and k with that log-sum-exp), against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_tile_amd import binding, workloads
from tests.parity_util import (LSE_BF16_MAX_ABS, assert_close, assert_grad_close, default_scale,
                               e4m3_codes, e4m3_descale, errors, to_gpu)

pytestmark = pytest.mark.gpu

CASES = [
    # name, volume, tile, windows per head
    ("hunyuan_tiles_2x2x3", (12, 16, 24), (6, 8, 8), [(6, 8, 8), (12, 16, 24), (6, 16, 8)]),
    ("tile64_3x4x4_w333", (12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 4, 4)]),
    ("tile48_ragged_runs", (9, 8, 12), (3, 4, 4), [(6, 4, 8), (9, 8, 12)]),
    ("tile128", (8, 8, 16), (4, 4, 8), [(4, 8, 8), (8, 4, 16)]),
    ("tile8_tiny", (4, 4, 6), (2, 2, 2), [(2, 2, 2), (4, 4, 6), (4, 2, 4)]),
    ("one_tile_volume", (6, 8, 8), (6, 8, 8), [(6, 8, 8)]),
    ("image_2d_tile8x8", (1, 32, 48), (1, 8, 8), [(1, 24, 24), (1, 32, 48), (1, 8, 16)]),
    ("padded_tile96", (7, 12, 20), (3, 4, 8), [(6, 8, 16), (9, 12, 24)]),
    ("padded_tile384", (13, 17, 19), (6, 8, 8), [(18, 24, 24)]),
]


def fp8_inputs(inp):
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    return e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd), qd, kd


def run_fp8(w, inp, q8, k8, qd, kd, order):
    """fp8 forward through the C ABI -> raster numpy output."""
    v = inp.v
    if order == "tile_major":
        q8, k8 = (oracle.to_tile_major(x, w.tile) for x in (q8, k8))
        v = oracle.to_tile_major(v, w.tile)
    q8g, k8g = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8))
    vg = to_gpu(v, "bf16")
    vol = w.volume if order == "tile_major" else None
    out = binding.sta_forward_fp8(q8g, k8g, vg, w.tile, inp.windows, qd, kd, volume=vol)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    if order == "tile_major":
        got = oracle.from_tile_major(got, w.volume, w.tile)
    return got


def run_fp8_lse(w, windows, v, q8, k8, qd, kd, order, scale):
    """fp8 forward with log-sum-exp through the C ABI -> (out, lse) as raster
    torch tensors (out bf16, lse float32); also checks that the output equals
    the forward without lse bit for bit (on the token rows: the padding rows
    of a tile-major output are left unwritten)."""
    if order == "tile_major":
        q8, k8 = (oracle.to_tile_major(x, w.tile) for x in (q8, k8))
        v = oracle.to_tile_major(v, w.tile)
    q8g, k8g = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8))
    vg = to_gpu(v, "bf16")
    vol = w.volume if order == "tile_major" else None
    out, lse = binding.sta_forward_fp8_lse(q8g, k8g, vg, w.tile, windows, qd, kd, scale=scale,
                                           volume=vol)
    plain = binding.sta_forward_fp8(q8g, k8g, vg, w.tile, windows, qd, kd, scale=scale,
                                    volume=vol)
    torch.cuda.synchronize()
    if order == "tile_major":
        raster = lambda x: torch.from_numpy(oracle.from_tile_major(x.float().cpu().numpy(), w.volume,
                                                                   w.tile)).to(torch.bfloat16).cuda()
        out, plain = raster(out), raster(plain)
        lse = torch.from_numpy(oracle.from_tile_major(lse.cpu().numpy()[..., None], w.volume,
                                                      w.tile)[..., 0]).cuda()
    assert torch.equal(out, plain), "output differs from the fp8 forward without lse"
    return out, lse


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fp8_forward_matches_oracle(case, order):
    name, volume, tile, windows = case
    w = workloads.small_case(volume, tile, windows, head_dim=128, dtype="bf16", seed=17, name=name)
    print(f"[case] fp8 forward {order} {w}", flush=True)
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    got = run_fp8(w, inp, q8, k8, qd, kd, order)
    ref = oracle.sta_attention_fp8(q8, k8, inp.v, tile, inp.windows, default_scale(128), qd, kd)
    assert_close(got, ref, "bf16", f"fp8 {name} {order}")


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: c[0])
def test_fp8_kernel_agrees_with_bf16_kernel_on_decoded_values(case):
    """Both kernels form exact products of the same values and sum them in
    float32; only the summation order and the rounding of a few probabilities
    to bf16 may differ."""
    name, volume, tile, windows = case
    w = workloads.small_case(volume, tile, windows, head_dim=128, dtype="bf16", seed=23, name=name)
    print(f"[case] fp8 vs bf16 kernel {w}", flush=True)
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    got = run_fp8(w, inp, q8, k8, qd, kd, "raster")
    qb = to_gpu(oracle.e4m3_decode(q8) * qd, "bf16")
    kb = to_gpu(oracle.e4m3_decode(k8) * kd, "bf16")
    out = binding.sliding_tile_attention(qb, kb, to_gpu(inp.v, "bf16"), tile, inp.windows)
    torch.cuda.synchronize()
    e = errors(got, out.float().cpu().numpy())
    print(f"[parity] fp8 vs bf16 kernel {name} {e}", flush=True)
    assert e["rel_l2"] <= 2e-3 and e["max_abs"] <= 1e-2, e


def test_fp8_large_scores_stay_stable():
    """Scores far from zero (the reference max moves often): the kernel keeps
    the same softmax as the oracle."""
    w = workloads.small_case((12, 16, 24), (6, 8, 8), [(6, 16, 16), (12, 16, 24)], head_dim=128,
                             dtype="bf16", seed=29, name="fp8_large")
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    scale = 4.0
    print(f"[case] fp8 large scores scale={scale}", flush=True)
    q8g, k8g = (torch.from_numpy(x).cuda() for x in (q8, k8))
    out = binding.sta_forward_fp8(q8g, k8g, to_gpu(inp.v, "bf16"), w.tile, inp.windows, qd, kd,
                                  scale=scale)
    torch.cuda.synchronize()
    ref = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, scale, qd, kd)
    assert_close(out.float().cpu().numpy(), ref, "bf16", "fp8 large scores")


def _tile_grid(volume, tile):
    """Tile coordinates (t, h, w) of every raster token, each (T, H, W)."""
    t, h, w = np.meshgrid(*(np.arange(n) // c for n, c in zip(volume, tile)), indexing="ij")
    return t, h, w


@pytest.mark.parametrize("order", ["raster", "tile_major"])
def test_fp8_key_scales_jumping_between_tiles(order):
    """Key magnitudes that change by up to 13x from tile to tile (full 64-key
    chunks, so the kernel that moves its reference max only on a lane-sum
    test): scores jump far past the lazy bound in both directions."""
    w = workloads.small_case((12, 16, 16), (4, 4, 4), [(8, 8, 8), (12, 16, 16)], head_dim=128,
                             dtype="bf16", seed=17, name="fp8_key_scale_jumps")
    print(f"[case] fp8 {w.name} {order}", flush=True)
    inp = workloads.make_inputs(w)
    t, h, x = _tile_grid(w.volume, w.tile)
    inp.k = inp.k * (1.0 + 3.0 * ((t * 7 + h * 3 + x) % 5))[None, None, :, :, :, None]
    q8, k8, qd, kd = fp8_inputs(inp)
    got = run_fp8(w, inp, q8, k8, qd, kd, order)
    ref = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, default_scale(128), qd, kd)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", f"{w.name} {order}")


@pytest.mark.parametrize("order", ["raster", "tile_major"])
def test_fp8_many_moderate_scores_move_the_reference_max(order):
    """Half the key tiles score about 5 (log2 units) above the others: single
    probabilities stay near 2^5, but lane sums of 16 of them pass 2^8, so the
    rescale has to come from the sum test."""
    d = 128
    w = workloads.small_case((8, 16, 16), (4, 4, 4), [(8, 8, 12)], head_dim=d, dtype="bf16",
                             seed=23, name="fp8_moderate_scores")
    print(f"[case] fp8 {w.name} {order}", flush=True)
    inp = workloads.make_inputs(w)
    scale = default_scale(d)
    alpha = 5.0 / (scale * math.log2(math.e))
    e0 = np.zeros(d, dtype=np.float32)
    e0[0] = 1.0
    t, h, x = _tile_grid(w.volume, w.tile)
    high = ((t + h + x) % 2).astype(np.float32)
    inp.q = alpha * e0 + 0.05 * inp.q
    inp.k = high[None, None, :, :, :, None] * e0 + 0.05 * inp.k
    q8, k8, qd, kd = fp8_inputs(inp)
    got = run_fp8(w, inp, q8, k8, qd, kd, order)
    ref = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, scale, qd, kd)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", f"{w.name} {order}")


def test_fp8_full_size_sampled_rows():
    w = workloads.STA_18_24_24
    print(f"[case] fp8 full size {w.name}: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    q8g, k8g = (torch.from_numpy(x).cuda() for x in (q8, k8))
    print(f"[case] fp8 full size {w.name}: running the raster kernel", flush=True)
    out = binding.sta_forward_fp8(q8g, k8g, to_gpu(inp.v, "bf16"), w.tile, inp.windows, qd, kd)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(w.B, w.heads, -1, w.head_dim)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(w.seed)
    n = oracle.tile_grid(w.volume, w.tile)
    n_tiles = n[0] * n[1] * n[2]
    interior = ((n[0] // 2) * n[1] + n[1] // 2) * n[2] + n[2] // 2
    tiles = sorted({0, n_tiles - 1, interior, int(rng.integers(0, n_tiles))})
    gots, refs = [], []
    for h in sorted({0, w.heads - 1, int(rng.integers(0, w.heads))}):
        rows = np.concatenate([rng.choice(oracle.tile_tokens(w.volume, w.tile, t), 8, replace=False)
                               for t in tiles])
        window = tuple(int(x) for x in inp.windows[h])
        ref = oracle.sta_attention_fp8_rows(q8, k8, inp.v, w.tile, window, default_scale(128),
                                            qd, kd, 0, h, rows)
        gots.append(got[0, h, rows])
        refs.append(ref)
    assert_close(np.concatenate(gots), np.concatenate(refs), "bf16", "fp8 full size samples")


def test_fp8_invalid_inputs_raise():
    w = workloads.small_case((4, 8, 8), (2, 4, 4), [(4, 8, 8)], head_dim=128, dtype="bf16", seed=1,
                             name="fp8_args")
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    q8g, k8g = (torch.from_numpy(x).cuda() for x in (q8, k8))
    v = to_gpu(inp.v, "bf16")
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(ValueError):
            binding.sta_forward_fp8(q8g, k8g, v, w.tile, inp.windows, bad, kd)
    w64 = workloads.small_case((4, 8, 8), (2, 4, 4), [(4, 8, 8)], head_dim=64, dtype="bf16", seed=1,
                               name="fp8_d64")
    i64 = workloads.make_inputs(w64)
    with pytest.raises(Exception):
        binding.sta_forward_fp8(torch.zeros(i64.q.shape, dtype=torch.uint8, device="cuda"),
                                torch.zeros(i64.q.shape, dtype=torch.uint8, device="cuda"),
                                to_gpu(i64.v, "bf16"), w64.tile, i64.windows, 1.0, 1.0)
    with pytest.raises(TypeError):
        binding.sta_forward_fp8(q8g.float(), k8g, v, w.tile, inp.windows, qd, kd)
    torch.cuda.synchronize()


LSE_CASES = [CASES[0], CASES[2], CASES[6], CASES[7]]


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", LSE_CASES, ids=lambda c: c[0])
def test_fp8_lse_matches_oracle(case, order):
    name, volume, tile, windows = case
    w = workloads.small_case(volume, tile, windows, head_dim=128, dtype="bf16", B=2, seed=31,
                             name=name)
    print(f"[case] fp8 forward with lse {order} {w}", flush=True)
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    scale = default_scale(128)
    out, lse = run_fp8_lse(w, inp.windows, inp.v, q8, k8, qd, kd, order, scale)
    ref = oracle.sta_lse_fp8(q8, k8, tile, inp.windows, scale, qd, kd)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref).max()
    print(f"[parity] fp8 {name} {order} lse max_abs {err:.3e}", flush=True)
    assert err <= LSE_BF16_MAX_ABS
    assert_close(out.float().cpu().numpy(),
                 oracle.sta_attention_fp8(q8, k8, inp.v, tile, inp.windows, scale, qd, kd), "bf16",
                 f"fp8 lse forward {name} {order}")


@pytest.mark.parametrize("order", ["raster", "tile_major"])
@pytest.mark.parametrize("case", LSE_CASES[:2] + LSE_CASES[3:], ids=lambda c: c[0])
def test_fp8_training_path_gradients(case, order):
    """fp8 scores in the forward, gradients from the bf16 backward on the
    decoded q and k (exact bf16 values) with the fp8 forward's out and lse:
    equal to the oracle's gradients of the attention on the decoded values
    (the fp8 rounding of q and k is taken as given, not differentiated)."""
    name, volume, tile, windows = case
    w = workloads.small_case(volume, tile, windows, head_dim=128, dtype="bf16", B=2, seed=37,
                             name=name)
    print(f"[case] fp8 training path {order} {w}", flush=True)
    inp = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    scale = default_scale(128)
    out, lse = run_fp8_lse(w, inp.windows, inp.v, q8, k8, qd, kd, order, scale)
    qdec, kdec = oracle.e4m3_decode(q8) * qd, oracle.e4m3_decode(k8) * kd
    q, k, v, do = (to_gpu(x, "bf16") for x in (qdec, kdec, inp.v, dout))
    assert torch.equal(q.double().cpu(), torch.from_numpy(qdec)), "decoded q is not a bf16 value"
    if order == "raster":
        grads = binding.sta_backward(q, k, v, out, do, lse, tile, inp.windows, scale)
    else:
        tmj = lambda x: binding.sta_reorder_tiles(x.contiguous(), tile)
        lse_t = binding.sta_reorder_tiles(lse.unsqueeze(-1).expand(*lse.shape, 4).contiguous(),
                                          tile)[..., 0].contiguous()
        g = binding.sta_backward(tmj(q), tmj(k), tmj(v), tmj(out), tmj(do), lse_t, tile,
                                 inp.windows, scale, volume=volume)
        grads = tuple(binding.sta_restore_order(x, volume, tile) for x in g)
    torch.cuda.synchronize()
    ref = oracle.sta_backward(qdec, kdec, inp.v, dout, tile, inp.windows, scale)
    for nm, g, r in zip(("dq", "dk", "dv"), grads, ref):
        assert_grad_close(g.float().cpu().numpy(), r, "bf16", f"fp8 path {name} {order} {nm}")


def test_fp8_lse_argument_errors():
    w = workloads.small_case((4, 8, 8), (2, 4, 4), [(4, 8, 8)], head_dim=128, dtype="bf16", seed=1,
                             name="fp8_lse_args")
    inp = workloads.make_inputs(w)
    q8, k8, qd, kd = fp8_inputs(inp)
    q8g, k8g = (torch.from_numpy(x).cuda() for x in (q8, k8))
    v = to_gpu(inp.v, "bf16")
    with pytest.raises(ValueError):   # lse of the wrong shape
        binding.sta_forward_fp8_lse(q8g, k8g, v, w.tile, inp.windows, qd, kd,
                                    lse=torch.empty(3, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):   # descale not positive
        binding.sta_forward_fp8_lse(q8g, k8g, v, w.tile, inp.windows, 0.0, kd)
    torch.cuda.synchronize()
