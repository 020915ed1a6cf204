"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import math

import numpy as np
import torch

# Output tolerances for bfloat16 inputs (fixed by the project's checking rule):
# max-abs <= 2e-2 and mean-abs <= 2e-3 against the float64 oracle. The
# relative-L2 bound is tighter and derived from the arithmetic: P and O are
# rounded to bf16 (relative error <= 2^-9 each), so a relative L2 error well
# under 1e-2 is expected.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_L2 = 1e-2
# float32 path: fp32 accumulation over at most ~1e5 keys; errors stay near
# 1e-6 in practice, 1e-4 leaves room for summation order.
F32_MAX_ABS = 1e-4
F32_REL_L2 = 1e-5


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_gpu(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=torch_dtype(dtype))


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    return {
        "max_abs": float(diff.max()),
        "mean_abs": float(diff.mean()),
        "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        "ref_std": float(ref.std()),
    }


def assert_close(got, ref, dtype: str, what: str = ""):
    e = errors(got, ref)
    print(f"[parity] {what} {e}", flush=True)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{what}: non-finite output"
    if dtype == "bf16":
        assert e["max_abs"] <= BF16_MAX_ABS, (what, e)
        assert e["mean_abs"] <= BF16_MEAN_ABS, (what, e)
        assert e["rel_l2"] <= BF16_REL_L2, (what, e)
    else:
        assert e["max_abs"] <= F32_MAX_ABS, (what, e)
        assert e["rel_l2"] <= F32_REL_L2, (what, e)
    return e


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# Gradient tolerances, relative to the reference (gradient magnitudes depend on
# the window size and the scale, so absolute bounds would mean nothing).
# bf16 path: the recomputed P and dS are rounded to bf16 before each matrix
# product and the gradients are rounded to bf16 (relative error <= 2^-9 each),
# so the relative L2 error stays well under 1e-2; single elements may lose
# more to cancellation, so their bound is relative to the largest element.
GRAD_BF16_REL_L2 = 1e-2
GRAD_BF16_MAX_REL = 2e-2
GRAD_F32_REL_L2 = 1e-5
GRAD_F32_MAX_REL = 1e-4
# Log-sum-exp: the bf16 forward sums the bf16-rounded probabilities (the
# values that multiply V), which moves lse by at most log(1 + 2^-9) < 2e-3.
LSE_BF16_MAX_ABS = 4e-3
LSE_F32_MAX_ABS = 1e-5
# Log-sum-exp-only passes (window recall), per row against the float64
# oracle. Nothing multiplies the probabilities there, so they are summed in
# fp32 without rounding, in both the dense and the window pass, for bf16 and
# float32 inputs alike. The error sources, for the small recall workloads
# (at most 4608 keys, 72 key chunks of 64 per row):
#   fp32 summation: each lane adds its chunk partials in order, then four lanes
#     combine: at most (n_chunks + 8) u = 80 * 2^-24 = 4.8e-6 relative;
#   exp2 argument: scale*log2(e) and the fma are rounded (relative u each) at
#     |argument| <= 8 above the reference max, and the hardware exp2 is within
#     about one ulp: well under 1e-6 relative on the probability-weighted sum;
#   score products: exact (bf16 x bf16, or fp32 in the fp32 kernel), summed in
#     fp32 over d <= 128 terms: typically a few 1e-7 on the scaled score;
#   storing lse in fp32: u |lse| < 1e-6 for |lse| < 16.
# Together under 1e-5; the bound leaves a factor two. Rounding the
# probabilities to bf16 before summing (the forward's rule, wrong here) moves
# these rows' lse by 2e-4 .. 1e-3 (tests/test_tolerances.py checks this on the
# recall workloads), so the bound tells the two apart.
LSE_FP32_SUM_MAX_ABS = 2e-5
# recall = mean_i exp(lse_window(i) - lse_full(i)) <= 1: both lse errors, the
# fp32 exp of the reduction (|argument| < 16, one ulp) and the fp32 result.
RECALL_MAX_ABS = 2 * LSE_FP32_SUM_MAX_ABS + 4 * 2.0 ** -24


def assert_grad_close(got, ref, dtype: str, what: str = ""):
    e = errors(got, ref)
    scale = float(np.abs(np.asarray(ref, dtype=np.float64)).max())
    e["max_abs_rel_to_max"] = e["max_abs"] / max(scale, 1e-300)
    print(f"[parity] {what} {e}", flush=True)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{what}: non-finite gradient"
    if dtype == "bf16":
        assert e["rel_l2"] <= GRAD_BF16_REL_L2, (what, e)
        assert e["max_abs_rel_to_max"] <= GRAD_BF16_MAX_REL, (what, e)
    else:
        assert e["rel_l2"] <= GRAD_F32_REL_L2, (what, e)
        assert e["max_abs_rel_to_max"] <= GRAD_F32_MAX_REL, (what, e)
    return e


# fp8 inputs (OCP E4M3 codes for q and k). The caller quantizes; here torch's
# own cast does it, after dividing by a power-of-two descale chosen so the
# largest magnitude stays below the format's 448 (no overflow to NaN).
def e4m3_descale(x: np.ndarray) -> float:
    amax = float(np.abs(np.asarray(x, dtype=np.float64)).max())
    return 2.0 ** math.ceil(math.log2(max(amax, 1e-30) / 448.0))


def e4m3_codes(x: np.ndarray, descale: float) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float64) / descale))
    return t.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
