"""Device transfers for the parity tests, plus the comparison rules of checks.py
(re-exported).  The rules, restated:

Indices: bit-exact, except for blocks whose oracle score lies within 1e-6 of
the k'-th best score of their row (several answers are then correct); lists
that differ only there are checked by recomputing the oracle attention on the
GPU's list.  Outputs: max |O_gpu - O_ref| <= 1e-2 and
||O_gpu - O_ref||_2 / ||O_ref||_2 <= 5e-3 (bf16 inputs, fp32 accumulation).
LSE: |LSE_gpu - LSE_ref| <= 1e-3 (natural log).  Threshold decisions: every
keep/skip choice of the GPU must match the fp64 walk replayed on the GPU's
own choices, unless the fp64 margin lies within THRESH_EPS of zero.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from checks import (LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, SCORE_TIE, THRESH_EPS, THRESH_STATS,  # noqa: F401
                    ambiguous, check_list, check_outputs, check_row_picks, check_threshold_walk, record_threshold)


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)
