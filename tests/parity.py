"""Comparison rules between the HIP path and the fp64 oracle.

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

SCORE_TIE = 1e-6
O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3
# Logit units; fp32 products of 128 bf16 terms with |logit| <= ~60 carry a
# rounding error far below this (about 1e-5); the band only has to absorb the
# fp32-vs-fp64 difference of max(tm - m).
THRESH_EPS = 1e-3


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def ambiguous(row: dict) -> set:
    """Non-forced candidates whose oracle score is within SCORE_TIE of the k'-th best."""
    if row["kth"] is None:
        return set()
    C, F, s = row["C"], set(row["F"].tolist()), row["s"]
    return {int(j) for j, sj in zip(C, s) if int(j) not in F and abs(sj - row["kth"]) <= SCORE_TIE}


def check_row_picks(gpu: np.ndarray, row: dict, where: str) -> int:
    """gpu: the row's picks padded with -1.  Returns the size of the tie band used."""
    g = set(int(x) for x in gpu if x >= 0)
    o = set(row["picks"].tolist())
    A = ambiguous(row)
    assert len(g) == len(o), f"{where}: {len(g)} picks vs oracle {len(o)}"
    assert g - A == o - A, f"{where}: picks differ outside the tie band: gpu-only {sorted(g - o)}, " \
                           f"oracle-only {sorted(o - g)}"
    return len(A)


def check_list(gpu_idx: np.ndarray, gpu_cnt: int, oracle_list: np.ndarray, band: set, where: str):
    g = gpu_idx[:gpu_cnt].astype(np.int64)
    assert np.all(np.diff(g) > 0), f"{where}: GPU list not strictly ascending"
    d = set(g.tolist()) ^ set(oracle_list.tolist())
    assert d <= band, f"{where}: lists differ outside the tie band: {sorted(d - band)}"


def check_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, lse_gpu=None, lse_ref=None, where=""):
    o_gpu, o_ref = np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{where}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)) if err.size else 0.0
    assert mx <= O_MAX_ABS, f"{where}: max abs err {mx:.3e} > {O_MAX_ABS}"
    assert rel <= O_REL_L2, f"{where}: rel L2 err {rel:.3e} > {O_REL_L2}"
    lmx = 0.0
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{where}: LSE finiteness differs"
        if fin.any():
            lmx = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max())
        assert lmx <= LSE_MAX_ABS, f"{where}: LSE max abs err {lmx:.3e}"
    return dict(max_abs=mx, rel_l2=rel, lse_max_abs=lmx)
