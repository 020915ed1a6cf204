"""The C-ABI library loads and exports what include/sta.h declares; host-side
argument checks reject bad calls before anything reaches a device. No test
here launches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sparse_attention_video_tile_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sta.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z ]+\*?\s*(sta_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_expected_functions():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.sta_abi_version() == binding.ABI_VERSION


def i3(*v):
    return binding._int_array(v)


def test_reorder_rejects_bad_arguments(lib):
    t = i3(6, 8, 8)
    assert lib.sta_reorder_tiles(None, FAKE, 1, 1, 128, 30, 48, 80, t, 0, None) == -1
    assert lib.sta_reorder_tiles(FAKE, FAKE * 4, 1, 1, 128, 30, 48, 80, i3(0, 8, 8), 0, None) == -1
    assert "tile" in binding.last_error()
    assert lib.sta_reorder_tiles(FAKE, FAKE * 4, 0, 1, 128, 30, 48, 80, t, 0, None) == -1
    assert lib.sta_reorder_tiles(FAKE, FAKE * 4, 1, 1, 128, 30, 48, 80, t, 7, None) == -1
    assert lib.sta_reorder_tiles(FAKE, FAKE * 4, 1, 1, 4, 30, 48, 80, t, 0, None) == -2
    # in-place / overlapping buffers
    assert lib.sta_reorder_tiles(FAKE, FAKE + 16, 1, 1, 128, 30, 48, 80, t, 0, None) == -1
    assert "overlap" in binding.last_error()
    assert lib.sta_restore_order(FAKE, FAKE, 1, 1, 128, 30, 48, 80, t, 0, None) == -1


def test_forward_rejects_bad_arguments(lib):
    t = i3(6, 8, 8)
    w = i3(18, 24, 24)
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, o=FAKE * 1000, B=1, heads=1, d=128,
                                  T=30, H=48, W=80, tile=t, win=w, scale=0.1, dt=0), **kw)

    def call(a):
        return lib.sta_forward(a["q"], a["k"], a["v"], a["o"], a["B"], a["heads"], a["d"], a["T"], a["H"],
                               a["W"], a["tile"], a["win"], a["scale"], a["dt"], None)

    assert call(args(q=None)) == -1
    assert call(args(o=None)) == -1
    assert call(args(win=None)) == -1
    assert call(args(heads=0)) == -1
    assert call(args(heads=binding.STA_MAX_HEADS + 1)) == -1
    assert call(args(win=i3(20, 24, 24))) == -1      # not whole tiles
    assert call(args(win=i3(36, 24, 24))) == -1      # larger than the volume
    assert "window" in binding.last_error()
    assert call(args(win=i3(0, 24, 24))) == -1
    assert call(args(tile=i3(7, 8, 8))) == -1        # the window is not whole tiles of 7
    assert call(args(win=i3(42, 24, 24), T=31)) == -1  # 7 tiles on a padded grid of 6
    assert call(args(scale=0.0)) == -1
    assert call(args(scale=float("nan"))) == -1
    assert call(args(scale=float("inf"))) == -1
    assert call(args(dt=5)) == -1
    assert call(args(d=96)) == -2
    assert call(args(q=FAKE + 8)) == -2              # misaligned
    assert call(args(o=FAKE * 2)) == -1              # out aliases k
    assert "overlap" in binding.last_error()


def test_full_attention_rejects_bad_arguments(lib):
    f = lib.sta_full_attention
    assert f(FAKE, FAKE * 2, FAKE * 3, None, 1, 1, 128, 1024, 0.1, 0, None) == -1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 1000, 1, 1, 128, 0, 0.1, 0, None) == -1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 1000, 1, 1, 128, 1024, -1.0, 0, None) == -1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 1000, 1, 1, 48, 1024, 0.1, 0, None) == -2
    # more heads than the work plan's per-head tables hold
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 1000, 1, binding.STA_MAX_HEADS + 1, 128, 1024, 0.1, 0,
             None) == -1
    assert "heads" in binding.last_error()


def test_kv_tiles_rejects_bad_arguments(lib):
    t = i3(6, 8, 8)
    w = i3(18, 24, 24)
    assert lib.sta_kv_tiles(None, FAKE, 1, 30, 48, 80, t, w, 27, None) == -1
    assert lib.sta_kv_tiles(FAKE, FAKE * 1000, 1, 30, 48, 80, t, w, 26, None) == -1  # max_kv too small
    assert lib.sta_kv_tiles(FAKE, FAKE + 4, 1, 30, 48, 80, t, w, 27, None) == -1  # overlap


@pytest.mark.parametrize(
    "heads,volume,tile,windows",
    [
        (1, (30, 48, 80), (6, 8, 8), [(18, 24, 24)]),
        (3, (30, 48, 80), (6, 8, 8), [(18, 24, 24), (30, 40, 40), (30, 48, 80)]),
        (2, (12, 16, 16), (4, 4, 4), [(12, 12, 12), (4, 8, 16)]),
        (1, (6, 9, 10), (3, 3, 2), [(3, 6, 4)]),
    ],
)
def test_kv_pair_count_matches_oracle(heads, volume, tile, windows):
    got = binding.sta_kv_pair_count(heads, volume, tile, windows)
    assert got == oracle.kv_pair_count(volume, tile, np.array(windows))


def test_kv_pair_count_rejects_bad_window(lib):
    assert lib.sta_kv_pair_count(1, 30, 48, 80, i3(6, 8, 8), i3(18, 24, 25)) == -1


def test_q_tiles_rejects_bad_arguments(lib):
    t = i3(6, 8, 8)
    w = i3(18, 24, 24)
    # the longest transposed list at this geometry: 5 x 4 x 4 = 80 query tiles
    # (the central key tile along t, of 5, is read by all 5 query tiles)
    longest = int(oracle.q_tile_lists((30, 48, 80), (6, 8, 8), [(18, 24, 24)])[1].max())
    assert longest == 80
    assert lib.sta_q_tiles(None, FAKE, 1, 30, 48, 80, t, w, 80, None) == -1
    assert lib.sta_q_tiles(FAKE, FAKE * 1000, 1, 30, 48, 80, t, w, 79, None) == -1
    assert "longest list 80" in binding.last_error()
    assert lib.sta_q_tiles(FAKE, FAKE + 4, 1, 30, 48, 80, t, w, 80, None) == -1


def test_forward_lse_rejects_bad_arguments(lib):
    t, w = i3(6, 8, 8), i3(18, 24, 24)
    f = lib.sta_forward_lse
    base = [FAKE, FAKE * 2, FAKE * 3, FAKE * 1000, FAKE * 5000, 1, 1, 128, 30, 48, 80, t, w, 0.1, 0]
    bad = list(base)
    bad[4] = None
    assert f(*bad, 0, None) == -1                     # lse NULL
    assert f(*base, 2, None) == -1                    # unknown order
    bad = list(base)
    bad[4] = FAKE * 2 + 64
    assert f(*bad, 1, None) == -1                     # lse overlaps k
    assert "overlap" in binding.last_error()


def test_forward_fp8_lse_rejects_bad_arguments(lib):
    """lse NULL, bad descales and head_dim are refused; lse is checked for
    overlap against q8 and k8 at one byte an element (an lse right after q8
    is accepted, and the call then fails on the overlapping output instead)."""
    t, w = i3(6, 8, 8), i3(18, 24, 24)
    f = lib.sta_forward_fp8_lse
    n = 30 * 48 * 80 * 128               # elements of one (b, h) tensor
    q8, k8, v = FAKE, FAKE + 4 * n, FAKE + 8 * n

    def call(lse, out=FAKE + 12 * n, d=128, qd=1.0, kd=1.0):
        return f(q8, k8, v, out, lse, 1, 1, d, 30, 48, 80, t, w, 0.1, qd, kd, 1, None)

    assert call(None) == -1
    assert call(FAKE + 16 * n, qd=0.0) == -1
    assert call(FAKE + 16 * n, kd=float("inf")) == -1
    assert call(FAKE + 16 * n, d=64) == binding.STA_ERR_UNSUPPORTED
    assert call(q8 + n - 64) == -1
    assert "lse overlaps" in binding.last_error()
    assert call(q8 + n, out=v + 64) == -1
    assert "output overlaps" in binding.last_error()


def test_window_recall_fp8_rejects_bad_arguments(lib):
    t = i3(6, 8, 8)
    cands = binding._int_array([18, 24, 24, 30, 48, 80])
    f = lib.sta_window_recall_fp8
    n = 30 * 48 * 80 * 128
    q8, k8, rec, ws = FAKE, FAKE + 4 * n, FAKE + 8 * n, FAKE + 12 * n

    def call(d=128, qd=1.0, kd=1.0, nc=2, order=1, ws=ws):
        return f(q8, k8, rec, ws, 1, 1, d, 30, 48, 80, t, cands, nc, 0.1, qd, kd, order, None)

    assert call(qd=-1.0) == -1
    assert call(kd=float("nan")) == -1
    assert call(d=64) == binding.STA_ERR_UNSUPPORTED
    assert call(nc=0) == -1
    assert call(order=3) == -1
    # the workspace is checked against q8 at one byte an element
    assert call(ws=q8 + n - 64) == -1
    assert "overlap" in binding.last_error()


def backward_args(**kw):
    a = dict(q=FAKE, k=FAKE * 2000, v=FAKE * 4000, o=FAKE * 6000, do=FAKE * 8000, lse=FAKE * 10000,
             dq=FAKE * 12000, dk=FAKE * 14000, dv=FAKE * 16000, delta=FAKE * 18000, B=1, heads=1,
             d=128, T=30, H=48, W=80, tile=i3(6, 8, 8), win=i3(18, 24, 24), scale=0.1, dt=0, order=0)
    a.update(kw)
    return a


def call_backward(lib, a):
    return lib.sta_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                            a["dv"], a["delta"], a["B"], a["heads"], a["d"], a["T"], a["H"], a["W"],
                            a["tile"], a["win"], a["scale"], a["dt"], a["order"], None)


def test_backward_rejects_bad_arguments(lib):
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "delta"):
        assert call_backward(lib, backward_args(**{name: None})) == -1, name
    assert call_backward(lib, backward_args(order=3)) == -1
    assert call_backward(lib, backward_args(win=i3(18, 24, 20))) == -1
    assert call_backward(lib, backward_args(d=96)) == -2
    assert call_backward(lib, backward_args(dt=4)) == -1
    assert call_backward(lib, backward_args(scale=-1.0)) == -1
    assert call_backward(lib, backward_args(dq=FAKE * 2000 + 256)) == -1    # dq overlaps k
    assert "overlap" in binding.last_error()
    assert call_backward(lib, backward_args(delta=FAKE * 14000 + 64)) == -1  # delta overlaps dk
    assert call_backward(lib, backward_args(dk=FAKE * 16000)) == -1          # dk aliases dv
    assert call_backward(lib, backward_args(q=FAKE + 8)) == -2               # misaligned
    # raster order: a whole-width window run of 10 tiles x 384 tokens fits, a
    # 1 x 1 x 8200-token run does not
    assert call_backward(lib, backward_args(order=1, T=1, H=1, W=8200, tile=i3(1, 1, 8),
                                            win=i3(1, 1, 8200), d=64)) == -2
    assert "raster order" in binding.last_error()


def raster_forward_rc(lib, tile, window, volume, d=64):
    """Return code of sta_forward_raster on never-dereferenced pointers: the
    host checks decide before any launch."""
    T, H, W = volume
    big = [(k + 1) << 40 for k in range(4)]
    return lib.sta_forward_raster(big[0], big[1], big[2], big[3], 1, 1, d, T, H, W, i3(*tile),
                                  i3(*window), 0.1, 0, None)


def test_raster_run_limit_is_the_library_s(lib):
    """Window runs of up to 8192 keys take the raster kernel; longer ones are
    refused with STA_ERR_UNSUPPORTED (the binding's fused path then reorders).
    The backward counts the transposed runs too: n_w = 4 tiles of 4096 with
    omega_w = 2 gives key tile 1 three query tiles (12288 keys)."""
    assert lib.sta_tile_list_len(1, 1, 1, 16384, i3(1, 1, 4096), i3(1, 1, 8192), 1) == 3
    assert lib.sta_tile_list_len(1, 1, 1, 16384, i3(1, 1, 4096), i3(1, 1, 8192), 0) == 2
    a = backward_args(order=1, T=1, H=1, W=16384, tile=i3(1, 1, 4096), win=i3(1, 1, 8192), d=64)
    assert call_backward(lib, a) == -2
    assert "12288" in binding.last_error()
    a = backward_args(order=1, T=1, H=1, W=8200, tile=i3(1, 1, 8), win=i3(1, 1, 8200), d=64)
    assert call_backward(lib, a) == -2


def test_tile_list_len_matches_oracle(lib):
    """The library's longest-list query, which sizes the list buffers, against
    the oracle's lists (forward and transposed), padded grids included."""
    for volume, tile, windows in [
        ((30, 48, 80), (6, 8, 8), [(18, 24, 24)]),
        ((30, 48, 80), (6, 8, 8), [(18, 24, 24), (30, 40, 40), (30, 48, 80)]),
        ((5, 6, 7), (2, 4, 4), [(4, 4, 4), (2, 8, 8), (6, 8, 8)]),
        ((1, 1, 16384), (1, 1, 4096), [(1, 1, 8192)]),
    ]:
        kv = oracle.kv_tile_lists(volume, tile, np.array(windows))[1].max()
        q = oracle.q_tile_lists(volume, tile, windows)[1].max()
        assert binding.sta_tile_list_len(len(windows), volume, tile, windows) == kv
        assert binding.sta_tile_list_len(len(windows), volume, tile, windows, transposed=True) == q
    t, w = i3(6, 8, 8), i3(18, 24, 24)
    assert lib.sta_tile_list_len(0, 30, 48, 80, t, w, 0) == -1
    assert lib.sta_tile_list_len(257, 30, 48, 80, t, w, 0) == -1
    assert lib.sta_tile_list_len(1, 30, 48, 80, t, i3(18, 24, 25), 0) == -1
    assert lib.sta_tile_list_len(1, 30, 48, 80, t, w, 2) == -1
    assert lib.sta_tile_list_len(1, 30, 48, 80, None, w, 0) == -1


def test_raster_frames_beyond_32bit_run_addressing_are_refused(lib):
    """One tile-row of frames (c_t * H * W tokens of up to 256 bytes) must fit
    the kernels' 32-bit offsets within a run: 2904 x 2904 frames do not, and
    the fused helper routes such volumes to the tile-major path."""
    t, w = i3(1, 8, 8), i3(1, 8, 8)
    big = [(k + 1) << 40 for k in range(4)]
    rc = lib.sta_forward_raster(big[0], big[1], big[2], big[3], 1, 1, 64, 1, 2904, 2904, t, w, 0.1, 0, None)
    assert rc == -2 and "addressing" in binding.last_error()
    assert raster_forward_rc(lib, (1, 8, 8), (1, 8, 8), (1, 2904, 2904)) == -2
    # 2896 x 2896 frames pass the raster checks: with misaligned pointers the
    # call gets as far as the alignment check (made after them)
    rc = lib.sta_forward_raster(FAKE + 8, FAKE * 100, FAKE * 200, FAKE * 300, 1, 1, 64, 1, 2896,
                                2896, t, w, 0.1, 0, None)
    assert rc == -2 and "aligned" in binding.last_error()


def test_window_recall_rejects_bad_arguments(lib):
    f = lib.sta_window_recall
    t = i3(6, 8, 8)
    cands = binding._int_array([18, 24, 24, 30, 40, 40])
    base = dict(q=FAKE, k=FAKE * 2000, r=FAKE * 4000, ws=FAKE * 6000, B=1, heads=2, d=128, T=30,
                H=48, W=80, tile=t, c=cands, n=2, scale=0.1, dt=0, order=1)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["r"], a["ws"], a["B"], a["heads"], a["d"], a["T"], a["H"],
                 a["W"], a["tile"], a["c"], a["n"], a["scale"], a["dt"], a["order"], None)

    assert call(q=None) == -1
    assert call(ws=None) == -1
    assert call(n=0) == -1
    assert call(order=7) == -1
    assert call(c=binding._int_array([18, 24, 24, 30, 40, 41])) == -1   # second candidate invalid
    assert "window" in binding.last_error()
    assert call(d=32) == -2
    assert call(ws=FAKE * 2000 + 64) == -1                              # workspace overlaps k
    assert "overlap" in binding.last_error()
    # the workspace holds n_candidates + 1 slots of B * heads * S floats: two
    # slots that end where k starts leave the third overlapping k
    slot = 1 * 2 * 30 * 48 * 80 * 4
    assert call(ws=FAKE * 2000 - 2 * slot) == -1
    assert "overlap" in binding.last_error()


def test_float32_attention_on_a_padded_grid_is_refused(lib):
    """Volume 5x6x7 with tile 2x4x4 is covered by a padded grid; float32
    attention refuses it before any launch, bf16 takes it (not launched here)."""
    t, w = i3(2, 4, 4), i3(4, 4, 4)
    rc = lib.sta_forward(FAKE, FAKE * 100, FAKE * 200, FAKE * 300, 1, 1, 64, 5, 6, 7, t, w, 0.1, 1, None)
    assert rc == -2 and "float32" in binding.last_error()
    rc = lib.sta_forward_raster(FAKE, FAKE * 100, FAKE * 200, FAKE * 300, 1, 1, 64, 5, 6, 7, t, w, 0.1, 1, None)
    assert rc == -2
    a = backward_args(T=5, H=6, W=7, tile=t, win=w, d=64, dt=1)
    assert call_backward(lib, a) == -2
    # a window larger than the padded grid is still invalid
    assert lib.sta_forward(FAKE, FAKE * 100, FAKE * 200, FAKE * 300, 1, 1, 64, 5, 6, 7, t,
                           i3(8, 4, 4), 0.1, 0, None) == -1


def call_backward_noalloc(lib, a):
    return lib.sta_backward_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                    a["dk"], a["dv"], a["B"], a["heads"], a["d"], a["T"], a["H"],
                                    a["W"], a["tile"], a["win"], a["scale"], a["dt"], a["order"], None)


def test_backward_noalloc_refuses_problems_beyond_its_scratch(lib):
    """The allocation-free backward keeps D in a static scratch of 8 Mi rows:
    72 heads of 115200 rows fit (the call then fails later, on the fake
    buffers' overlap), 73 do not, and it says so before anything is enqueued."""
    for heads, msg in ((73, "scratch"), (72, "overlap")):
        win = binding._int_array([18, 24, 24] * heads)   # one window per head
        assert call_backward_noalloc(lib, backward_args(heads=heads, win=win, order=1)) == -1
        assert msg in binding.last_error()
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert call_backward_noalloc(lib, backward_args(**{name: None})) == -1, name
    assert call_backward_noalloc(lib, backward_args(order=3)) == -1
