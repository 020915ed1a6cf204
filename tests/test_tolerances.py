"""CPU checks that the GPU tests' tolerances are tight enough to see the
mistakes they are meant to catch. Each plants the mistake in the oracle (on
the CPU) and checks that the planted result falls outside the bound."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sta_backward_oracle
from sparse_attention_video_tile_amd import workloads
from tests.parity_util import LSE_FP32_SUM_MAX_ABS
from tests.test_gpu_recall import CASES as RECALL_CASES


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def _softmax_rows_bf16_p(q_rows, k_all, allowed, scale):
    """The planted mistake: probabilities rounded to bf16 before the row sum
    (what the forward does for P V, wrong for a log-sum-exp-only pass)."""
    s = scale * (q_rows @ k_all.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(allowed, _bf16(np.exp(s - m)), 0.0)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


@pytest.mark.parametrize("case", RECALL_CASES, ids=lambda c: c[0])
def test_lse_only_bound_sees_bf16_rounded_probabilities(case, monkeypatch):
    name, volume, tile, cands, heads, d, dtype = case
    w = workloads.small_case(volume, tile, [cands[0]] * heads, head_dim=d, dtype=dtype, B=2,
                             seed=31, name=name, sinusoid_amp=0.5)
    inp = workloads.make_inputs(w)
    scale = 1.0 / math.sqrt(d)
    windows = (volume, cands[-1])   # the two passes the GPU test compares row by row
    exact = [oracle.sta_lse(inp.q, inp.k, tile, [win] * heads, scale) for win in windows]
    monkeypatch.setattr(sta_backward_oracle, "_softmax_rows", _softmax_rows_bf16_p)
    planted = [oracle.sta_lse(inp.q, inp.k, tile, [win] * heads, scale) for win in windows]
    for a, b in zip(exact, planted):
        assert np.abs(a - b).max() > 3 * LSE_FP32_SUM_MAX_ABS
