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
