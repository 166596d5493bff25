"""Worker for the full-size threshold-prefill parity check: walks the sampled
query tiles of one KV group in the fp64 oracle.  It runs in a spawned process
that imports numpy, the oracle and the input generators only, never the GPU."""
from __future__ import annotations

import numpy as np

import synth
from checks import check_threshold_walk


def _f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def check_group(task: dict):
    """task: k, v (bf16 bits, [L, D]), tile, lam, scale, causal and items, each
    dict(h, qt, q (bf16 bits of the tile's rows), dec {kv_tile: bool}, kept,
    o (fp32 [rows, D]), lse).  Returns (decisions, flips, replays, max flip margin)."""
    k, v = _f64(task["k"]), _f64(task["v"])
    L, T = k.shape[0], task["tile"]
    tot = [0, 0, 0, 0.0]
    for it in task["items"]:
        qt = it["qt"]
        rows = np.arange(qt * T, min((qt + 1) * T, L))
        d, f, r, m = check_threshold_walk(_f64(it["q"]), k, v, rows, T, task["lam"], task["scale"], task["causal"],
                                          it["dec"], it["kept"], it["o"].astype(np.float64), it["lse"],
                                          f"thr h{it['h']} qt{qt}")
        tot[0] += d
        tot[1] += f
        tot[2] += r
        tot[3] = max(tot[3], m)
    return tuple(tot), len(task["items"])
