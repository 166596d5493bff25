"""Comparison rules between the HIP path and the fp64 oracle (numpy only, so
that worker processes which never touch the GPU can use them).

Indices: bit-exact, except for blocks whose oracle score lies within 1e-6 of
the k'-th best score of their row (several answers are then correct); lists
that differ only there are checked by recomputing the oracle attention on the
GPU's list.  Outputs: max |O_gpu - O_ref| <= 1e-2 and
||O_gpu - O_ref||_2 / ||O_ref||_2 <= 5e-3 (bf16 inputs, fp32 accumulation).
LSE: |LSE_gpu - LSE_ref| <= 1e-3 (natural log).  Threshold decisions: every
keep/skip choice of the GPU must match the fp64 walk replayed on the GPU's
own choices, unless the fp64 margin lies within THRESH_EPS of zero; the
choices inside the band that went the other way ("flips") and the walks
replayed are counted in THRESH_STATS and printed at the end of the session.
"""
from __future__ import annotations

import numpy as np

import oracle as orc

SCORE_TIE = 1e-6
O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3
# Logit units (natural log).  A margin is max(tm - m) - ln(lambda), with tm and m
# maxima of fp32 dot products of 128 bf16 products; at |logit| <= ~60 their
# rounding error is about 1e-5, so a band of 1e-4 holds it with room.
THRESH_EPS = 1e-4
THRESH_STATS = {"decisions": 0, "flips": 0, "walks": 0, "replays": 0, "max_flip_margin": 0.0}


def record_threshold(decisions: int, flips: int, walks: int, replays: int, max_flip_margin: float):
    THRESH_STATS["decisions"] += int(decisions)
    THRESH_STATS["flips"] += int(flips)
    THRESH_STATS["walks"] += int(walks)
    THRESH_STATS["replays"] += int(replays)
    THRESH_STATS["max_flip_margin"] = max(THRESH_STATS["max_flip_margin"], float(max_flip_margin))


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


def check_threshold_walk(q_rows, k, v, rows, tile, lam, scale, causal, dec, kept_count, o_gpu, lse_gpu, where):
    """One (head, query tile) of threshold prefill.  The oracle walks it with its
    own decisions; if the GPU's keep map (dec, {kv_tile: bool}) differs, the first
    difference (tiles are visited from the highest index down) must sit within
    THRESH_EPS of the fp64 threshold, the walk is replayed on the GPU's choices,
    and each replayed choice must agree with the fp64 margin outside the band.
    Outputs are compared with the walk that was followed.
    Returns (decisions, flips, replayed, max |margin| of a flip)."""
    args = (q_rows, k, v, rows, tile, lam, scale, causal)
    r = orc.threshold_walk(*args, masses=False)
    replayed = r["decision"] != dec
    flips, fmax = 0, 0.0
    if replayed:
        first = max(j for j in dec if dec[j] != r["decision"][j])
        assert abs(r["margin"][first]) <= THRESH_EPS, \
            f"{where} tile {first}: gpu keep={dec[first]}, fp64 margin {r['margin'][first]:.4g}"
        r = orc.threshold_walk(*args, decisions=dec, masses=False)
    for j, mg in r["margin"].items():
        if dec[j] != (mg >= 0):
            assert abs(mg) <= THRESH_EPS, f"{where} tile {j}: gpu keep={dec[j]}, fp64 margin {mg:.4g}"
            flips += 1
            fmax = max(fmax, abs(mg))
    assert kept_count == len(r["kept"]), f"{where}: kept {kept_count} vs walk {len(r['kept'])}"
    check_outputs(o_gpu, r["O"], lse_gpu, r["lse"], where)
    return len(dec), flips, int(replayed), fmax
