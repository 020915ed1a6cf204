"""CPU oracle for STA with fp8 queries and keys -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module. It shares no code with the HIP library and never calls it.

The pages mention FP8 quantization inside a sparse attention kernel (dianyo
ICML2025 blog, Sparse VideoGen, "Observation & Proposed Method") without
fixing a format or where it applies. Readings taken here:

* Format: OCP 8-bit floating point, E4M3 (the "OFP8" specification): sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
  subnormals m/8 * 2^-6; no infinities; the codes with every exponent and
  mantissa bit set (0x7F, 0xFF) are NaN; the largest finite value is 448.
* Placement: queries and keys are fp8 with one positive descale per tensor,
  so the score of query i and key j is
      scale * (q_descale * Q8_i) . (k_descale * K8_j),
  and the values V stay bf16. The attention itself is the STA definition of
  ``sta_oracle`` on the decoded values, in float64.
"""

from __future__ import annotations

import numpy as np

from .sta_backward_oracle import sta_lse, window_recall
from .sta_oracle import sta_attention, sta_attention_rows


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of OCP E4M3 codes (any integer array of bytes 0..255)."""
    c = np.asarray(codes).astype(np.int64)
    if c.size and (c.min() < 0 or c.max() > 255):
        raise ValueError("E4M3 codes are bytes")
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    subnormal = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


def sta_attention_fp8(q8, k8, v, tile, windows, scale, q_descale, k_descale) -> np.ndarray:
    """STA output (float64, raster order) for fp8 code tensors q8, k8 of shape
    (B, heads, T, H, W, d), per-tensor descales, and v of the same shape."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    if not (np.all(np.isfinite(q)) and np.all(np.isfinite(k))):
        raise ValueError("NaN code in q8 or k8")
    return sta_attention(q, k, np.asarray(v, dtype=np.float64), tile, windows, scale)


def sta_attention_fp8_rows(q8, k8, v, tile, window, scale, q_descale, k_descale, b: int, h: int,
                           query_tokens) -> np.ndarray:
    """Selected raster output rows of ``sta_attention_fp8`` for batch b, head h
    (decodes only that head)."""
    q = e4m3_decode(q8[b:b + 1, h:h + 1]) * float(q_descale)
    k = e4m3_decode(k8[b:b + 1, h:h + 1]) * float(k_descale)
    vv = np.asarray(v[b:b + 1, h:h + 1], dtype=np.float64)
    return sta_attention_rows(q, k, vv, tile, window, scale, 0, 0, query_tokens)


def sta_lse_fp8(q8, k8, tile, windows, scale, q_descale, k_descale) -> np.ndarray:
    """Row log-sum-exp (float64, raster order, shape (B, heads, T, H, W)) of the
    STA scores on the decoded fp8 values, scale * (q_descale Q8_i) .
    (k_descale K8_j), over each row's window keys: the probabilities a
    fixed-window backward pass recomputes from (atlas.scime.ai summary,
    "Approach": fine-tuning with the window fixed)."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    if not (np.all(np.isfinite(q)) and np.all(np.isfinite(k))):
        raise ValueError("NaN code in q8 or k8")
    return sta_lse(q, k, tile, windows, scale)


def window_recall_fp8(q8, k8, tile, candidates, scale, q_descale, k_descale) -> np.ndarray:
    """Attention recall (float64, (B, heads, n_candidates)) of each candidate
    window for the scores on the decoded fp8 values (podcast transcript, the
    answer on attention recall): the oracle's recall on those values."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    if not (np.all(np.isfinite(q)) and np.all(np.isfinite(k))):
        raise ValueError("NaN code in q8 or k8")
    return window_recall(q, k, tile, candidates, scale)
