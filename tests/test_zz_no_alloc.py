"""GPU: the allocation-free backward (sta_backward_noalloc, D in the library's
static device scratch) against sta_backward (caller-owned D workspace),
called through the C ABI: two calls in a row, the second on a smaller
problem, then a third in the other token order. The kernels are the same, so
the gradients must be identical bit for bit."""

import ctypes

import pytest
import torch

from sparse_attention_video_tile_amd import binding

pytestmark = pytest.mark.gpu


def _draw(shape, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return [torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype) for _ in range(4)]


def _noalloc_c_call(q, k, v, out, dout, lse, grads, tile, windows, scale, dtype_code, volume, order):
    lib = binding.load_library()
    B, heads = q.shape[:2]
    d = q.shape[-1]
    T, H, W = volume
    rc = lib.sta_backward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), B, heads, d, T, H, W,
        binding._int_array(tile), binding._int_array([x for w in windows for x in w]),
        ctypes.c_float(scale), dtype_code, order,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, binding.last_error()


# (volume, tile, windows per head, B, head_dim, dtype, order)
CALLS = [
    ((30, 48, 80), (6, 8, 8), [(18, 24, 24), (30, 40, 40)], 1, 128, torch.bfloat16, "raster"),
    ((12, 16, 24), (6, 8, 8), [(6, 8, 8), (12, 16, 24), (6, 16, 8)], 2, 128, torch.bfloat16, "raster"),
    ((5, 6, 7), (2, 4, 4), [(4, 4, 4), (6, 8, 8)], 2, 64, torch.bfloat16, "tile_major"),
    ((12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 8, 4)], 1, 64, torch.float32, "raster"),
]


def test_noalloc_backward_equals_backward_on_consecutive_calls():
    for i, (volume, tile, windows, B, d, dtype, order) in enumerate(CALLS):
        print(f"[case] no-alloc backward call {i}: volume {volume} tile {tile} windows {windows} "
              f"B={B} d={d} {dtype} {order}", flush=True)
        heads = len(windows)
        q, k, v, dout = _draw((B, heads) + tuple(volume) + (d,), dtype, 100 + i)
        vol = None
        if order == "tile_major":
            q, k, v, dout = (binding.sta_reorder_tiles(x, tile) for x in (q, k, v, dout))
            vol = volume
        scale = 1.0 / d ** 0.5
        out, lse = binding.sta_forward_lse(q, k, v, tile, windows, scale, volume=vol)
        ref = binding.sta_backward(q, k, v, out, dout, lse, tile, windows, scale, volume=vol)
        grads = [torch.full_like(q, float("nan")) for _ in range(3)]
        _noalloc_c_call(q, k, v, out, dout, lse, grads, tile, windows, scale,
                        binding.STA_BF16 if dtype == torch.bfloat16 else binding.STA_F32, volume,
                        binding.STA_TILE_MAJOR if order == "tile_major" else binding.STA_RASTER)
        torch.cuda.synchronize()
        for nm, a, r in zip(("dq", "dk", "dv"), grads, ref):
            if order == "tile_major":   # padding rows are not gradients: compare the real ones
                a, r = (binding.sta_restore_order(x, volume, tile) for x in (a, r))
            assert torch.equal(a, r), f"call {i} {nm}: max diff {(a.float() - r.float()).abs().max()}"
        print(f"[parity] no-alloc call {i}: dq, dk, dv identical to sta_backward", flush=True)
