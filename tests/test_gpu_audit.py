"""GPU: synchronisation audit of the attention pipeline.

The forward kernels stream K and V through two LDS buffers: the loads of
chunk it+1 are in flight while chunk it is computed, ordered by one wait and
one barrier per chunk. libsta_audit.so is the same source built with a single
buffer, whose next chunk is loaded only after every wave has finished the
current one (no overlap to get wrong). The arithmetic and its order are the
same, so the outputs must be identical bit for bit; a missing wait or
barrier in the double-buffered pipeline would show as a difference. Checked
at the 30x48x80 headline workload and on the other kernel variants (tile-
major, per-head windows, ragged runs, padded grids, fp8, log-sum-exp only,
dense)."""

import math
import os

import pytest
import torch

from sparse_attention_video_tile_amd import binding, build, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def audit_lib():
    if not os.path.exists(build.AUDIT_LIB):
        pytest.fail(f"{build.AUDIT_LIB} is missing: build the package first")
    return binding.open_library(build.AUDIT_LIB)


def with_lib(lib, fn, *args, **kw):
    """Run a binding call against another build of the library."""
    binding.load_library()
    saved = binding._lib
    binding._lib = lib
    try:
        return fn(*args, **kw)
    finally:
        binding._lib = saved


def draw(B, heads, volume, d, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shape = (B, heads) + tuple(volume) + (d,)
    return [torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype) for _ in range(3)]


CASES = [
    # name, B, volume, tile, windows per head, d
    ("headline_30x48x80_w18x24x24", 1, (30, 48, 80), (6, 8, 8), [(18, 24, 24)] * 24, 128),
    ("mixed_heads_30x48x80", 1, (30, 48, 80), (6, 8, 8),
     [tuple(x) for x in workloads.head_windows(workloads.MIXED_HEADS).tolist()], 128),
    ("ragged_tile48", 2, (9, 8, 12), (3, 4, 4), [(3, 4, 4), (6, 4, 8)], 128),
    ("padded_tile32_d64", 2, (5, 6, 7), (2, 4, 4), [(4, 4, 4), (2, 8, 8), (6, 8, 8)], 64),
    ("padded_tile384", 2, (13, 17, 19), (6, 8, 8), [(18, 24, 24)], 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_single_buffer_equals_double_buffer(audit_lib, case):
    name, B, volume, tile, windows, d = case
    print(f"[case] audit {name}", flush=True)
    q, k, v = draw(B, len(windows), volume, d, 17)
    a = binding.sta_forward_raster(q, k, v, tile, windows)
    b = with_lib(audit_lib, binding.sta_forward_raster, q, k, v, tile, windows)
    qt, kt, vt = (binding.sta_reorder_tiles(x, tile) for x in (q, k, v))
    # padding rows of a tile-major output are left unwritten: compare the
    # tokens (restored to raster order)
    c = binding.sta_restore_order(binding.sta_forward(qt, kt, vt, volume, tile, windows), volume, tile)
    e = binding.sta_restore_order(with_lib(audit_lib, binding.sta_forward, qt, kt, vt, volume, tile, windows),
                                  volume, tile)
    torch.cuda.synchronize()
    assert torch.equal(a, b), f"{name} raster: {(a.float() - b.float()).abs().max().item()}"
    assert torch.equal(c, e), f"{name} tile-major: {(c.float() - e.float()).abs().max().item()}"
    print(f"[parity] audit {name}: raster and tile-major identical to the single-buffer build", flush=True)
    if d == 128:
        codes = []
        for x in (q, k):
            amax = float(x.float().abs().max())
            ds = 2.0 ** math.ceil(math.log2(amax / 448.0))
            codes.append(((x.float() / ds).to(torch.float8_e4m3fn).view(torch.uint8), ds))
        (q8, qd), (k8, kd) = codes
        f = binding.sta_forward_fp8(q8, k8, v, tile, windows, qd, kd)
        h = with_lib(audit_lib, binding.sta_forward_fp8, q8, k8, v, tile, windows, qd, kd)
        torch.cuda.synchronize()
        assert torch.equal(f, h), f"{name} fp8"
    if volume[0] * volume[1] * volume[2] <= 4096:
        cands = [windows[0], tuple(volume)] if all(x % c == 0 for x, c in zip(volume, tile)) else [windows[0]]
        r1 = binding.sta_window_recall(q, k, tile, cands)
        r2 = with_lib(audit_lib, binding.sta_window_recall, q, k, tile, cands)
        S = volume[0] * volume[1] * volume[2]
        qd_, kd_, vd_ = (x.reshape(B, len(windows), S, d) for x in (q, k, v))
        d1 = binding.sta_full_attention(qd_, kd_, vd_)
        d2 = with_lib(audit_lib, binding.sta_full_attention, qd_, kd_, vd_)
        torch.cuda.synchronize()
        assert torch.equal(r1, r2), f"{name} recall"
        assert torch.equal(d1, d2), f"{name} dense"
