"""Pins for the fp8 oracle (CPU): the E4M3 decoder against the format's fixed
values and torch's own float8_e4m3fn type, and the fp8 attention and its row
log-sum-exp against closed forms, invariants of the descales and library
routines."""

import math

import numpy as np
import scipy.special
import torch

import oracle
from sparse_attention_video_tile_amd import workloads
from tests.parity_util import e4m3_codes, e4m3_descale


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(lib[ok]))


def test_e4m3_values_fixed_by_the_format():
    d = oracle.e4m3_decode
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0
    assert d(0x3C) == 1.5
    assert d(0x40) == 2.0
    assert d(0xC0) == -2.0
    assert d(0x7E) == 448.0                # largest finite
    assert d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x78) == 256.0                # exponent field 15 is a normal binade


def test_e4m3_positive_codes_increase_and_mirror():
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    # the subnormal spacing continues unchanged into the first binade
    assert pos[0x08] - pos[0x07] == pos[0x07] - pos[0x06] == 2.0 ** -9
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF))
    assert np.array_equal(neg, -pos)


def _case(seed=5):
    w = workloads.small_case((4, 8, 8), (2, 4, 4), [(4, 8, 8), (2, 4, 4)], head_dim=128,
                             dtype="bf16", seed=seed, name="fp8_pin")
    return w, workloads.make_inputs(w)


def test_zero_queries_give_the_window_mean_of_v():
    w, inp = _case()
    q8 = np.zeros(inp.q.shape, dtype=np.uint8)
    kd = e4m3_descale(inp.k)
    k8 = e4m3_codes(inp.k, kd)
    out = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, 0.1, 1.0, kd)
    vf = inp.v.astype(np.float64).reshape(w.B, w.heads, -1, 128)
    of = out.reshape(w.B, w.heads, -1, 128)
    toks = np.arange(vf.shape[2])
    for h in range(w.heads):
        mask = oracle.token_mask_rows(w.volume, w.tile, tuple(inp.windows[h]), toks)
        want = (mask.astype(np.float64) @ vf[0, h]) / mask.sum(axis=1, keepdims=True)
        assert np.allclose(of[0, h], want, rtol=0, atol=1e-12)


def test_descales_fold_into_the_scale_and_commute():
    w, inp = _case(seed=9)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 1.0 / math.sqrt(128)
    a = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, s, qd, kd)
    b = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, s * qd * kd, 1.0, 1.0)
    c = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, s, kd, qd)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert np.allclose(a, c, rtol=0, atol=1e-12)
    # a coarse check that the quantized scores stay near the bf16 ones
    ref = oracle.sta_attention(inp.q, inp.k, inp.v, w.tile, inp.windows, s)
    assert np.abs(a - ref).max() < 0.1


def test_whole_volume_window_equals_library_attention():
    volume, tile = (2, 4, 4), (1, 2, 2)
    w = workloads.small_case(volume, tile, [volume], head_dim=128, dtype="bf16", seed=3,
                             name="fp8_dense_pin")
    inp = workloads.make_inputs(w)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 0.125
    out = oracle.sta_attention_fp8(q8, k8, inp.v, tile, inp.windows, s, qd, kd)
    qt = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64) * qd
    kt = torch.from_numpy(k8).view(torch.float8_e4m3fn).to(torch.float64) * kd
    vt = torch.from_numpy(inp.v.astype(np.float64))
    sh = (w.B, w.heads, -1, 128)
    lib = torch.nn.functional.scaled_dot_product_attention(
        qt.reshape(sh), kt.reshape(sh), vt.reshape(sh), scale=s).numpy()
    assert np.allclose(out.reshape(sh), lib, rtol=0, atol=1e-12)


def test_row_subsets_match_whole_fp8_output():
    """The row-subset fp8 entry point (the checker of the sampled full-size
    fp8 test) slices one (b, h) before decoding; it must give the matching rows
    of the whole output for every (b, h) of a B = 2, three-head draw with a
    different window per head, descales included."""
    w = workloads.small_case((4, 8, 8), (2, 4, 4), [(4, 8, 8), (2, 4, 4), (2, 8, 4)], head_dim=128,
                             dtype="bf16", B=2, seed=13, name="fp8_rows_pin")
    inp = workloads.make_inputs(w)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 1.0 / math.sqrt(128)
    full = oracle.sta_attention_fp8(q8, k8, inp.v, w.tile, inp.windows, s, qd, kd)
    rows = np.array([0, 9, 63, 130, 255])
    for b in range(w.B):
        for h in range(w.heads):
            part = oracle.sta_attention_fp8_rows(q8, k8, inp.v, w.tile, tuple(inp.windows[h]), s,
                                                 qd, kd, b, h, rows)
            np.testing.assert_allclose(part, full[b, h].reshape(-1, 128)[rows], rtol=1e-12,
                                       atol=1e-14)


def test_lse_fp8_zero_queries_give_log_of_window_size():
    """All scores zero: every row's log-sum-exp is the log of its window's key
    count (a closed form independent of the keys and the descales)."""
    w, inp = _case()
    q8 = np.zeros(inp.q.shape, dtype=np.uint8)
    kd = e4m3_descale(inp.k)
    k8 = e4m3_codes(inp.k, kd)
    lse = oracle.sta_lse_fp8(q8, k8, w.tile, inp.windows, 0.3, 2.0, kd)
    toks = np.arange(int(np.prod(w.volume)))
    for h in range(w.heads):
        counts = oracle.token_mask_rows(w.volume, w.tile, tuple(inp.windows[h]), toks).sum(axis=1)
        assert np.allclose(lse[0, h].reshape(-1), np.log(counts), rtol=0, atol=1e-12)


def test_lse_fp8_whole_volume_equals_scipy_logsumexp():
    """Whole-volume window: the row log-sum-exp over every key, computed with
    scipy on values decoded by torch's float8_e4m3fn type."""
    volume, tile = (2, 4, 4), (1, 2, 2)
    w = workloads.small_case(volume, tile, [volume, volume], head_dim=128, dtype="bf16", seed=5,
                             name="fp8_lse_dense_pin")
    inp = workloads.make_inputs(w)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 0.125
    lse = oracle.sta_lse_fp8(q8, k8, tile, inp.windows, s, qd, kd)
    qt = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64).numpy() * qd
    kt = torch.from_numpy(k8).view(torch.float8_e4m3fn).to(torch.float64).numpy() * kd
    for h in range(w.heads):
        qf, kf = qt[0, h].reshape(-1, 128), kt[0, h].reshape(-1, 128)
        want = scipy.special.logsumexp(s * qf @ kf.T, axis=1)
        assert np.allclose(lse[0, h].reshape(-1), want, rtol=0, atol=1e-12)


def test_lse_fp8_descales_fold_into_the_scale_and_commute():
    w, inp = _case(seed=11)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 1.0 / math.sqrt(128)
    a = oracle.sta_lse_fp8(q8, k8, w.tile, inp.windows, s, qd, kd)
    b = oracle.sta_lse_fp8(q8, k8, w.tile, inp.windows, s * qd * kd, 1.0, 1.0)
    c = oracle.sta_lse_fp8(q8, k8, w.tile, inp.windows, s, kd, qd)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert np.allclose(a, c, rtol=0, atol=1e-12)


def test_recall_fp8_closed_forms():
    """Zero query codes: every key gets the same full-attention probability,
    so a window keeps its share of the keys; the whole volume keeps all of it;
    nested windows keep more."""
    w, inp = _case()
    kd = e4m3_descale(inp.k)
    k8 = e4m3_codes(inp.k, kd)
    q8 = np.zeros(inp.q.shape, dtype=np.uint8)
    cands = [(2, 4, 4), (4, 4, 4), (4, 8, 8)]
    r = oracle.window_recall_fp8(q8, k8, w.tile, cands, 0.2, 1.0, kd)
    S = int(np.prod(w.volume))
    toks = np.arange(S)
    for c, win in enumerate(cands):
        share = oracle.token_mask_rows(w.volume, w.tile, win, toks).sum() / (S * S)
        assert np.allclose(r[0, :, c], share, rtol=0, atol=1e-12)
    qd = e4m3_descale(inp.q)
    q8 = e4m3_codes(inp.q, qd)
    r = oracle.window_recall_fp8(q8, k8, w.tile, cands, 1.0 / math.sqrt(128), qd, kd)
    assert np.allclose(r[..., 2], 1.0, rtol=0, atol=1e-12)
    assert np.all(r[..., 0] < r[..., 1]) and np.all(r[..., 1] < r[..., 2])


def test_recall_fp8_is_the_recall_of_torch_decoded_values():
    """The fp8 recall equals the recall definition evaluated directly, with
    scipy, on values decoded by torch's float8_e4m3fn type: the mean over
    rows of the full softmax mass on the window's keys."""
    w, inp = _case(seed=7)
    qd, kd = e4m3_descale(inp.q), e4m3_descale(inp.k)
    q8, k8 = e4m3_codes(inp.q, qd), e4m3_codes(inp.k, kd)
    s = 1.0 / math.sqrt(128)
    win = (2, 4, 4)
    r = oracle.window_recall_fp8(q8, k8, w.tile, [win], s, qd, kd)
    qt = torch.from_numpy(q8).view(torch.float8_e4m3fn).to(torch.float64).numpy() * qd
    kt = torch.from_numpy(k8).view(torch.float8_e4m3fn).to(torch.float64).numpy() * kd
    toks = np.arange(int(np.prod(w.volume)))
    mask = oracle.token_mask_rows(w.volume, w.tile, win, toks)
    for h in range(w.heads):
        sc = s * qt[0, h].reshape(-1, 128) @ kt[0, h].reshape(-1, 128).T
        p = np.exp(sc - scipy.special.logsumexp(sc, axis=1, keepdims=True))
        assert np.allclose(r[0, h, 0], (p * mask).sum(axis=1).mean(), rtol=0, atol=1e-12)
