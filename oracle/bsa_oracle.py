"""fp64 reference for query-aware block-sparse attention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use this
module.  It imports nothing from the HIP library and shares no helper, table or
constant with it.  Every array argument is float64 holding exactly the values
handed to the GPU (bf16 or fp32 upcast without change).

Sources (cited by page title and section; no code is printed on the pages):
  [LoSA]  "LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
          Language Models", technical summary sec. 1 (Problem) and sec. 2
          (Methodology: locality pruning, reuse for stable tokens, sparse
          attention for active tokens, shrinking the KV union).
  [Prism] "Prism: Spectral-Aware Block-Sparse Attention", technical summary
          sec. 1-3 (mean pooling as low-pass filter; dual-band estimation;
          energy-based temperature calibration).
  [NSA]   "Native Sparse Attention: Hardware-Aligned and Natively Trainable
          Sparse Attention" (news article), section on the three-branch NSA
          structure (selection block 64, 16 blocks incl. 1 initial + 2 local)
          and the section on GQA/MQA-compatible memory access.
  [FASA]  "FASA: Frequency-aware Sparse Attention", technical summary sec. 2
          (FC functional sparsity: high frequency = low dims; FAC keeps the
          original absolute positions).
  [BLASST] "BLASST: Dynamic BLocked Attention Sparsity via Softmax
          Thresholding", technical summary sec. 2 (skip a block when its local
          max trails the running max by more than ln(lambda); skip exp, V load
          and PV for it).

Readings of points the pages leave open are marked READING; each is listed
with its reason in the design notes.  Pins (independent checks of this module)
live in tests/test_oracle_pins.py.  Parity unpinned: the exact group-score
aggregation (sum of per-head softmax probabilities) and the temperature
formula are readings with no independent ground truth beyond the invariances
and special cases tested there.
"""
from __future__ import annotations

import math

import numpy as np

ROPE_HALF = 0
ROPE_INTERLEAVED = 1
TAU_FLOOR = 1e-6


# ------------------------------------------------------------------ bands ---
def fast_band_mask(D: int, layout: int) -> np.ndarray:
    """Boolean mask over head dims: True for the fast-rotating (high-frequency) band.

    [FASA] sec. 2 and [Prism] sec. 3: RoPE rotates 2-D frequency chunks; low FC
    index = high frequency = positional/local information, high FC index = low
    frequency = semantic information.  READING: the band split is at FC D/4
    (half of the chunks on each side).  With the rotate-half layout FC i owns
    dims i and i + D/2; with the interleaved layout it owns dims 2i and 2i+1.
    """
    fc_of_dim = np.empty(D, dtype=np.int64)
    for d in range(D):
        if layout == ROPE_HALF:
            fc_of_dim[d] = d if d < D // 2 else d - D // 2
        elif layout == ROPE_INTERLEAVED:
            fc_of_dim[d] = d // 2
        else:
            raise ValueError(layout)
    return fc_of_dim < D // 4


# -------------------------------------------------------------- summaries ---
def block_summaries(x: np.ndarray, block: int, layout: int = ROPE_HALF):
    """Mean-pooled block summaries and per-band mean energies.

    [Prism] sec. 1-2: a block is represented by the mean of its vectors.  For
    block j with tokens T_j = [j*b, min((j+1)*b, L)):
        mean_j   = (1/|T_j|) sum_t x_t
        energy_j = (1/|T_j|) sum_t ||x_t[band]||^2   for band in (fast, slow)
    A ragged last block averages only its valid tokens.
    x: [..., L, D]  ->  mean [..., NB, D], energy [..., NB, 2]
    """
    L, D = x.shape[-2], x.shape[-1]
    NB = -(-L // block)
    fast = fast_band_mask(D, layout)
    mean = np.zeros(x.shape[:-2] + (NB, D))
    energy = np.zeros(x.shape[:-2] + (NB, 2))
    for j in range(NB):
        seg = x[..., j * block:min((j + 1) * block, L), :]
        n = seg.shape[-2]
        mean[..., j, :] = seg.sum(axis=-2) / n
        sq = seg * seg
        energy[..., j, 0] = sq[..., fast].sum(axis=(-2, -1)) / n
        energy[..., j, 1] = sq[..., ~fast].sum(axis=(-2, -1)) / n
    return mean, energy


def retained_fraction(mean: np.ndarray, energy: np.ndarray, layout: int) -> np.ndarray:
    """rho per (.., band): energy of the pooled means over the mean energy of the tokens.

    [Prism] sec. 2: pooling RoPE'd vectors cancels fast-rotating chunks; rho is
    the share of a band's energy that survives pooling, summed over all blocks.
    A band with zero token energy keeps rho = 1.
    """
    D = mean.shape[-1]
    fast = fast_band_mask(D, layout)
    num = np.stack([(mean[..., fast] ** 2).sum(axis=(-2, -1)),
                    (mean[..., ~fast] ** 2).sum(axis=(-2, -1))], axis=-1)
    den = energy.sum(axis=-2)
    out = np.ones_like(num)
    ok = den > 0
    out[ok] = num[ok] / den[ok]
    return out


def band_temperatures(k_mean, k_energy, layout: int, G: int, q_mean=None, q_energy=None) -> np.ndarray:
    """Per-(batch, query head, band) temperature tau; shape [B, Hq, 2].

    READING of [Prism] sec. 3 ("energy-based temperature calibration": pooling
    weakens each band's magnitude by a computable amount and a per-band
    temperature restores it; no formula is printed).  A pooled logit
    qbar . kbar shrinks in amplitude by sqrt(rho_Q) * sqrt(rho_K), so
        tau[b, h, band] = max(1e-6, sqrt(rho_Q[b, h, band] * rho_K[b, h // G, band]))
    with rho_Q = 1 when queries are not pooled.
    """
    rk = retained_fraction(k_mean, k_energy, layout)            # [B, Hkv, 2]
    B, Hkv = rk.shape[:2]
    rk_h = np.repeat(rk, G, axis=1)                               # [B, Hq, 2]
    if q_mean is not None:
        rq = retained_fraction(q_mean, q_energy, layout)
    else:
        rq = np.ones_like(rk_h)
    return np.maximum(TAU_FLOOR, np.sqrt(rq * rk_h))


# ---------------------------------------------------------- candidates ---
def candidate_blocks(qb: int, NB: int, p: dict, Lq: int) -> np.ndarray:
    """KV blocks a query block may select.

    Non-causal (decode / denoise over a prefix): all NB blocks.  Causal:
    blocks whose first key is visible to the last row of the query block.
    """
    if not p["causal"]:
        return np.arange(NB)
    last_row = min((qb + 1) * p["q_block"], Lq) - 1
    jmax = min(NB - 1, (p["q_pos0"] + last_row) // p["kv_block"])
    return np.arange(jmax + 1)


def forced_blocks(C: np.ndarray, p: dict) -> np.ndarray:
    """[NSA] selection setting: the initial block(s) and the most recent block(s)
    are always kept.  For causal prefill the most recent candidate is the
    diagonal block."""
    n = len(C)
    f = set(C[:min(p["n_first"], n)].tolist())
    if p["n_last"] > 0:
        f |= set(C[max(0, n - p["n_last"]):].tolist())
    return np.array(sorted(f), dtype=np.int64)


def num_scored_picks(n_cand: int, n_forced: int, p: dict) -> int:
    """k' scored picks beyond the forced blocks.

    Fixed budget ``topk``, or, when ``topk_num`` > 0, ceil(topk_num * |C| /
    topk_den) (READING of "about 10% of causal blocks": an exact integer
    ceiling).  Capped by the number of non-forced candidates.
    """
    if p.get("topk_num", 0) > 0:
        k = -(-(p["topk_num"] * n_cand) // p["topk_den"])
    else:
        k = p["topk"]
    return int(min(k, n_cand - n_forced))


# -------------------------------------------------------------- scoring ---
def _softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - z.max())
    return e / e.sum()


def group_scores(qrows: np.ndarray, kmean: np.ndarray, scale: float, tau=None, fast=None) -> np.ndarray:
    """Group score of each candidate block for one selection row.

    qrows: [G, D] the row's query (or pooled query) for each head of the KV
    group; kmean: [n_cand, D] pooled keys of the candidates.
    Single band ([Prism] sec. 1 baseline, mean-pooled key scoring):
        z_h = scale * q_h . kbar_j,   p_h = softmax_j z_h
    Dual band ([Prism] sec. 3; tau: [G, 2], fast: band mask):
        z_h^band = scale * q_h[band] . kbar_j[band] / tau_h^band
        p_h = (softmax_j z_h^fast + softmax_j z_h^slow) / 2
    READING: the selection is shared by the GQA group ([NSA] section on
    GQA/MQA-aware access) and the group score is s_j = sum_h p_h[j].
    """
    s = np.zeros(kmean.shape[0])
    for h in range(qrows.shape[0]):
        if tau is None:
            s += _softmax(scale * (kmean @ qrows[h]))
        else:
            zf = scale * (kmean[:, fast] @ qrows[h, fast]) / tau[h, 0]
            zs = scale * (kmean[:, ~fast] @ qrows[h, ~fast]) / tau[h, 1]
            s += 0.5 * (_softmax(zf) + _softmax(zs))
    return s


def top_picks(s: np.ndarray, C: np.ndarray, F: np.ndarray, kprime: int):
    """F plus the k' best non-forced candidates by score (ties: lower block index).

    Returns (sorted unique picks, k'-th best non-forced score or None when
    every non-forced candidate is taken).
    """
    free = ~np.isin(C, F)
    cj, cs = C[free], s[free]
    order = np.lexsort((cj, -cs))          # score descending, then index ascending
    chosen = cj[order[:kprime]]
    kth = float(cs[order[kprime - 1]]) if 0 < kprime < len(cj) else None
    return np.union1d(F, chosen).astype(np.int64), kth


def select_blocks(p: dict, k_mean: np.ndarray, q: np.ndarray | None = None, q_mean: np.ndarray | None = None,
                  tau: np.ndarray | None = None, row_mask: np.ndarray | None = None, Lq: int | None = None):
    """Per-(batch, KV group, query block) sorted list of selected KV blocks.

    Raw mode (decode, denoise): ``q`` [B, Hq, Lq, D]; every row of a query block
    is a selection row.  Pooled mode (prefill): ``q_mean`` [B, Hq, NQB, D]; the
    pooled query is the block's single selection row ([Prism] sec. 3: purely
    block-level estimation).
    Each selection row picks F + top-k' of the remaining candidates; the list
    of a query block is the union of its (unmasked) rows' picks ([LoSA] sec. 1:
    memory traffic is set by the union over the block; sec. 2: selecting only
    for active rows shrinks it).  READING: every row of the block then attends
    to the whole union.
    Returns dict(lists[b][g][qb] -> int array, rows[(b, g, row)] -> dict).
    """
    B, Hkv, NB, D = k_mean.shape
    pooled = q is None
    Hq = (q_mean if pooled else q).shape[1]
    G = Hq // Hkv
    if pooled:
        NQB = q_mean.shape[2]
        Lq = Lq if Lq is not None else NQB * p["q_block"]
    else:
        Lq = q.shape[2]
        NQB = -(-Lq // p["q_block"])
    fast = fast_band_mask(D, p["layout"]) if p.get("dual_band") else None
    lists = [[[None] * NQB for _ in range(Hkv)] for _ in range(B)]
    rows = {}
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            for qb in range(NQB):
                C = candidate_blocks(qb, NB, p, Lq)
                F = forced_blocks(C, p)
                kp = num_scored_picks(len(C), len(F), p)
                if pooled:
                    sel_rows = [(qb, q_mean[b, hs, qb, :])]
                else:
                    r0, r1 = qb * p["q_block"], min((qb + 1) * p["q_block"], Lq)
                    sel_rows = [(r, q[b, hs, r, :]) for r in range(r0, r1)
                                if row_mask is None or row_mask[b, r]]
                union = np.zeros(0, dtype=np.int64)
                for r, qr in sel_rows:
                    t = None if tau is None else tau[b, hs, :]
                    s = group_scores(qr, k_mean[b, g, C, :], p["scale"], t, fast)
                    picks, kth = top_picks(s, C, F, kp)
                    rows[(b, g, r)] = dict(C=C, F=F, s=s, kth=kth, picks=picks, kprime=kp)
                    union = np.union1d(union, picks)
                lists[b][g][qb] = union.astype(np.int64)
    return dict(lists=lists, rows=rows, NQB=NQB, G=G)


# ------------------------------------------------------------ attention ---
def attend_tokens(q: np.ndarray, k: np.ndarray, v: np.ndarray, toks: np.ndarray, scale: float,
                  q_pos: np.ndarray | None = None):
    """Exact softmax attention of rows q [R, D] over keys/values k[toks], v[toks].

    ``q_pos`` (optional, [R]) masks keys whose absolute position exceeds the
    row's position (causal).  LSE = ln sum exp(scale * q . k) (natural log,
    scale included).  A row that sees no key gets O = 0 and LSE = -inf.
    """
    R, D = q.shape
    O = np.zeros((R, v.shape[1]))
    lse = np.full(R, -np.inf)
    if len(toks) == 0:
        return O, lse
    S = scale * (q @ k[toks].T)
    if q_pos is not None:
        S = np.where(toks[None, :] <= q_pos[:, None], S, -np.inf)
    m = S.max(axis=1)
    ok = np.isfinite(m)
    P = np.exp(S[ok] - m[ok, None])
    l = P.sum(axis=1)
    O[ok] = (P @ v[toks]) / l[:, None]
    lse[ok] = m[ok] + np.log(l)
    return O, lse


def block_tokens(blocks: np.ndarray, block: int, L: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min((j + 1) * block, L)) for j in blocks]).astype(np.int64)


def sparse_attention(p: dict, q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, row_mask=None,
                     qblocks=None, heads=None):
    """Attention of each query row over the tokens of its query block's list.

    [FASA] sec. 2 (FAC): full-dimension attention restricted to the selected
    tokens, at their original absolute positions.  Equals dense attention with
    -inf logits outside the selection.  Rows with row_mask = 0 are left out
    (their entries stay NaN here; the library leaves them untouched, [LoSA]
    sec. 2 reuse for stable tokens).
    Returns O [B, Hq, Lq, D], LSE [B, Hq, Lq] (NaN where not computed).
    """
    B, Hq, Lq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    NQB = -(-Lq // p["q_block"])
    O = np.full((B, Hq, Lq, v.shape[3]), np.nan)
    LSE = np.full((B, Hq, Lq), np.nan)
    for b in range(B):
        for qb in (range(NQB) if qblocks is None else qblocks):
            r0, r1 = qb * p["q_block"], min((qb + 1) * p["q_block"], Lq)
            rows = np.array([r for r in range(r0, r1) if row_mask is None or row_mask[b, r]], dtype=np.int64)
            if len(rows) == 0:
                continue
            qpos = (p["q_pos0"] + rows) if p["causal"] else None
            for h in (range(Hq) if heads is None else heads):
                g = h // G
                toks = block_tokens(lists[b][g][qb], p["kv_block"], L)
                o, lse = attend_tokens(q[b, h, rows], k[b, g], v[b, g], toks, p["scale"], qpos)
                O[b, h, rows] = o
                LSE[b, h, rows] = lse
    return O, LSE


def window_decode(p: dict, q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, window: int, gates=None):
    """Selected blocks plus a sliding window ([NSA] structure section: parallel
    branches over the selected blocks and a sliding window of w tokens, w = 512;
    the compression branch needs learned weights and is left out).

    Decode rows (q_block = 1): row r sits at position q_pos0 + r; its window is
    the ``window`` keys ending there (fewer near the start).  Each branch is its
    own exact softmax; READING: the branch outputs are summed with the given
    gates [B, Hq, Lq, 2] (a model's gate values; 1 and 1 when None).
    Returns O [B, Hq, Lq, D] and LSE [B, Hq, Lq, 2] (list branch, window branch).
    """
    B, Hq, Lq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O_sel, L_sel = sparse_attention(p, q, k, v, lists)
    O_win = np.zeros_like(O_sel)
    L_win = np.zeros_like(L_sel)
    for b in range(B):
        for h in range(Hq):
            for r in range(Lq):
                hi = min(L, p["q_pos0"] + r + 1)
                toks = np.arange(max(0, hi - window), hi)
                o, l = attend_tokens(q[b, h, [r]], k[b, h // G], v[b, h // G], toks, p["scale"])
                O_win[b, h, r], L_win[b, h, r] = o[0], l[0]
    g = np.ones((B, Hq, Lq, 2)) if gates is None else gates
    O = g[..., 0:1] * O_sel + g[..., 1:2] * O_win
    return O, np.stack([L_sel, L_win], axis=-1)


# ------------------------------------------------- token-level importance ---
def fc_dims(f: int, D: int, layout: int) -> np.ndarray:
    """The two dims of frequency chunk f ([FASA] sec. 2: RoPE rotates each
    chunk's pair of dims together): (f, f + D/2) in the rotate-half layout,
    (2f, 2f + 1) in the interleaved one."""
    return np.array([f, f + D // 2]) if layout == ROPE_HALF else np.array([2 * f, 2 * f + 1])


def token_scores(q: np.ndarray, k: np.ndarray, fc_mask: np.ndarray, layout: int) -> np.ndarray:
    """[FASA] sec. 2, token importance prediction: each head scores every token
    by q . k over the dims of its dominant chunks only (fc_mask [Hq, D/2],
    given; the offline calibration that picks them is out of scope).
    q [B, Hq, 1, D], k [B, Hkv, L, D] -> scores [B, Hq, L]."""
    B, Hq, _, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    S = np.zeros((B, Hq, L))
    for h in range(Hq):
        fs = np.nonzero(fc_mask[h])[0]
        dims = np.concatenate([fc_dims(f, D, layout) for f in fs]) if len(fs) else np.zeros(0, dtype=np.int64)
        for b in range(B):
            S[b, h] = k[b, h // G][:, dims] @ q[b, h, 0, dims]
    return S


def top_tokens(s: np.ndarray, budget: int):
    """The min(budget, L) best tokens of one head by score, ties to the lower
    token, in ascending token order; also the score of the last one taken."""
    n = min(budget, len(s))
    order = sorted(range(len(s)), key=lambda t: (-s[t], t))[:n]
    return np.sort(np.array(order, dtype=np.int64)), s[order[-1]]


def token_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, scale: float):
    """[FASA] sec. 2, focused attention: each head attends with all dims to its
    own tokens at their original positions.  lists[b][h] -> token array.
    Returns O [B, Hq, 1, D], LSE [B, Hq, 1]."""
    B, Hq, _, D = q.shape
    G = Hq // k.shape[1]
    O = np.zeros((B, Hq, 1, v.shape[3]))
    LSE = np.zeros((B, Hq, 1))
    for b in range(B):
        for h in range(Hq):
            O[b, h], LSE[b, h] = attend_tokens(q[b, h], k[b, h // G], v[b, h // G], np.asarray(lists[b][h]), scale)
    return O, LSE


# ------------------------------------------------------- locality pruning ---
def active_rows(q_cur: np.ndarray, q_prev: np.ndarray, theta: float):
    """[LoSA] sec. 2, locality pruning: a row is active when the mean squared
    change of its query vector between denoising steps (over heads and dims)
    exceeds theta.  READING: the query change stands in for the hidden-state
    change.  The comparison is taken in float32, the kernel's precision.
    q_cur, q_prev: [B, H, R, D] -> (mask bool [B, R], mse float64 [B, R])
    """
    d = q_cur - q_prev
    mse = (d * d).mean(axis=(1, 3))
    mask = mse.astype(np.float32) > np.float32(theta)
    return mask, mse


# ------------------------------------------------- full denoising step ---
def merge_states(O_a: np.ndarray, L_a: np.ndarray, O_b: np.ndarray, L_b: np.ndarray):
    """Attention state over the union of two disjoint key sets from the states
    over each: [LoSA] sec. 2 keeps a stable token's prefix-attention output and
    statistics, which combine with the attention over the block's own keys.

    Softmax over a disjoint union: with weights w_x = e^(L_x - L) and
    L = ln(e^L_a + e^L_b), O = w_a O_a + w_b O_b.  An LSE of -inf is an empty
    set, whose O is ignored; both empty gives O = 0, L = -inf.
    O_x [..., D], L_x [...] (natural log).
    """
    m = np.maximum(L_a, L_b)
    L = np.full(m.shape, -np.inf)
    ok = np.isfinite(m)
    with np.errstate(invalid="ignore"):                # -inf - -inf where both sides are empty (masked)
        wa = np.where(np.isfinite(L_a), np.exp(np.where(ok, L_a - m, 0.0)), 0.0)
        wb = np.where(np.isfinite(L_b), np.exp(np.where(ok, L_b - m, 0.0)), 0.0)
    tot = wa + wb
    L[ok] = m[ok] + np.log(tot[ok])
    fa = np.where(ok, wa / np.where(ok, tot, 1.0), 0.0)[..., None]
    fb = np.where(ok, wb / np.where(ok, tot, 1.0), 0.0)[..., None]
    O = np.where(fa > 0, fa * np.nan_to_num(O_a), 0.0) + np.where(fb > 0, fb * np.nan_to_num(O_b), 0.0)
    return O, L


def block_self_attention(q: np.ndarray, kb: np.ndarray, vb: np.ndarray, scale: float):
    """Attention of the block's R rows over the block's own R keys, in both
    directions (a block-wise diffusion LM denoises all tokens of the block
    together; READING: no causal mask inside the block).
    q [B, Hq, R, D]; kb, vb [B, Hkv, R, D] -> O [B, Hq, R, D], LSE [B, Hq, R]."""
    B, Hq, R, D = q.shape
    G = Hq // kb.shape[1]
    O = np.zeros((B, Hq, R, vb.shape[3]))
    LSE = np.zeros((B, Hq, R))
    toks = np.arange(kb.shape[2])
    for b in range(B):
        for h in range(Hq):
            O[b, h], LSE[b, h] = attend_tokens(q[b, h], kb[b, h // G], vb[b, h // G], toks, scale)
    return O, LSE


def denoise_step(p: dict, q: np.ndarray, k: np.ndarray, v: np.ndarray, kb: np.ndarray, vb: np.ndarray, lists,
                 row_mask, cache_O: np.ndarray, cache_L: np.ndarray):
    """One denoising step of a block ([LoSA] sec. 2).

    Rows with row_mask set (all rows when it is None: the dense first step,
    whose lists hold every prefix block) recompute their prefix attention over
    their block's list; the others keep the cached prefix state.  Every row
    then merges its prefix state with the attention over the block's own keys.
    Returns O, LSE (the step's output) and the updated prefix cache.
    """
    O_p, L_p = sparse_attention(p, q, k, v, lists, row_mask=row_mask)
    upd = np.ones(q.shape[2], dtype=bool)[None, :].repeat(q.shape[0], 0) if row_mask is None else row_mask
    cO = np.where(upd[:, None, :, None], O_p, cache_O)
    cL = np.where(upd[:, None, :], L_p, cache_L)
    O_b, L_b = block_self_attention(q, kb, vb, p["scale"])
    O, L = merge_states(cO, cL, O_b, L_b)
    return O, L, cO, cL


# ---------------------------------------------------- threshold attention ---
def threshold_walk(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows_pos: np.ndarray, tile: int, lam: float,
                   scale: float, causal: bool = True, decisions: dict | None = None, masses: bool = True):
    """One (head, query tile) of softmax-threshold attention ([BLASST] sec. 2).

    q: [T, D] rows of the tile at absolute positions rows_pos; k, v: [L, D].
    KV tiles are visited from the last one the tile can see down to tile 0
    (READING: diagonal first, then descending; the pages give no order).  For
    each visited tile: S = scale * q k^T (causal-masked), tm_r = max over the
    tile of S[r, :].  Row r votes to keep the tile when tm_r is finite and
    either m_r is still -inf or tm_r - m_r >= ln(lambda).  The tile is kept
    when any row votes keep (READING: one all-or-nothing decision per tile for
    the rows that share it); a kept tile updates m_r = max(m_r, tm_r), a
    skipped tile leaves m unchanged and contributes nothing.  lambda = 0 never
    skips.  Output = exact softmax over the kept tiles' visible keys.

    ``decisions`` (optional, {kv_tile: bool}) replays another implementation's
    keep/skip choices; the margins are still computed on this walk's state so
    the caller can check that every replayed choice agrees with fp64 except
    within a rounding band.
    Returns dict(O [T, D], lse [T], kept [tiles], order, margin {tile: float},
    decision {tile: bool}, mass_kept, mass_skipped); ``masses=False`` leaves the
    two masses None (a second pass over the keys, not needed for O and LSE).
    """
    L = k.shape[0]
    ln_lam = math.log(lam) if lam > 0 else -math.inf
    last_pos = int(rows_pos.max())
    jmax = (min(L - 1, last_pos) // tile) if causal else (-(-L // tile) - 1)
    T = q.shape[0]
    m = np.full(T, -np.inf)
    kept, margin, decision = [], {}, {}
    for j in range(jmax, -1, -1):
        c0, c1 = j * tile, min((j + 1) * tile, L)
        S = scale * (q @ k[c0:c1].T)
        if causal:
            S = np.where(np.arange(c0, c1)[None, :] <= rows_pos[:, None], S, -np.inf)
        tm = S.max(axis=1)
        fin = np.isfinite(tm)
        if np.any(fin & ~np.isfinite(m)):
            mg = math.inf
        elif np.any(fin):
            mg = float(np.max(tm[fin] - m[fin])) - ln_lam
        else:
            mg = -math.inf
        keep = mg >= 0
        margin[j] = mg
        if decisions is not None:
            keep = bool(decisions[j])
        decision[j] = keep
        if keep:
            m = np.maximum(m, tm)
            kept.append(j)
    toks = block_tokens(np.array(sorted(kept), dtype=np.int64), tile, L)
    O, lse = attend_tokens(q, k, v, toks, scale, rows_pos if causal else None)
    if not masses:
        return dict(O=O, lse=lse, kept=sorted(kept), margin=margin, decision=decision, mass_kept=None,
                    mass_skipped=None)
    # exp-mass kept vs skipped (for the skipped-mass bound), per row, relative to the final max
    all_toks = block_tokens(np.arange(jmax + 1), tile, L)
    S_all = scale * (q @ k[all_toks].T)
    if causal:
        S_all = np.where(all_toks[None, :] <= rows_pos[:, None], S_all, -np.inf)
    mx = S_all.max(axis=1, keepdims=True)
    E = np.exp(S_all - mx)
    kept_tok = np.isin(all_toks // tile, np.array(kept, dtype=np.int64))
    return dict(O=O, lse=lse, kept=sorted(kept), margin=margin, decision=decision,
                mass_kept=E[:, kept_tok].sum(axis=1), mass_skipped=E[:, ~kept_tok].sum(axis=1))


def threshold_attention(p: dict, q: np.ndarray, k: np.ndarray, v: np.ndarray, pairs, q_pos0: int = 0):
    """Run ``threshold_walk`` for the (b, h, q_tile) triples in ``pairs``."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    T = p["tile"]
    Lq = q.shape[2]
    out = {}
    for (b, h, qt) in pairs:
        r0, r1 = qt * T, min((qt + 1) * T, Lq)
        out[(b, h, qt)] = threshold_walk(q[b, h, r0:r1], k[b, h // G], v[b, h // G], q_pos0 + np.arange(r0, r1),
                                         T, p["lam"], p["scale"], bool(p["causal"]))
    return out


def threshold_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, lam: float, scale: float, tile: int,
                     decisions: np.ndarray | None = None):
    """Softmax-threshold decode ([BLASST] sec. 2, decode kernel: the same skip
    rule, where the saving is the V load of a skipped block).

    q [B, Hq, 1, D]; k, v [B, Hkv, L, D]; the query sees every key.  Each query
    head walks the whole sequence with ``threshold_walk`` on its single row:
    tiles of ``tile`` keys from the newest down (READING, as for prefill), its
    own running max, the rule of the pages.  A tile's V is needed when any head
    of its KV group keeps it.
    ``decisions`` (optional, [B, Hq, ntiles] bool) replays another
    implementation's choices, as in ``threshold_walk``.
    Returns O [B, Hq, 1, D], LSE [B, Hq, 1], keep [B, Hq, ntiles] bool and
    margin [B, Hq, ntiles] (this walk's tm - m - ln(lambda) per tile).
    """
    B, Hq, _, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    nt = -(-L // tile)
    O = np.zeros((B, Hq, 1, v.shape[3]))
    LSE = np.zeros((B, Hq, 1))
    keep = np.zeros((B, Hq, nt), dtype=bool)
    margin = np.zeros((B, Hq, nt))
    for b in range(B):
        for h in range(Hq):
            dec = None if decisions is None else {j: bool(decisions[b, h, j]) for j in range(nt)}
            r = threshold_walk(q[b, h], k[b, h // G], v[b, h // G], np.array([L - 1]), tile, lam, scale,
                               causal=False, decisions=dec)
            keep[b, h, r["kept"]] = True
            for j, mg in r["margin"].items():
                margin[b, h, j] = mg
            O[b, h, 0] = r["O"][0]
            LSE[b, h, 0] = r["lse"][0]
    return O, LSE, keep, margin


# ------------------------------------------------------------ decode step ---
def decode_step(p: dict, q: np.ndarray, k: np.ndarray, v: np.ndarray, k_mean: np.ndarray, k_energy: np.ndarray):
    """One GQA decode step: refresh the newest block's summary, select, attend.

    k_mean / k_energy hold the summaries of the prefix (updated in place for
    the last block).  Returns (O, LSE, lists).
    """
    L = k.shape[2]
    b = p["kv_block"]
    j = (L - 1) // b
    m, e = block_summaries(k[:, :, j * b:min((j + 1) * b, L), :], b, p["layout"])
    k_mean[:, :, j, :] = m[:, :, 0, :]
    k_energy[:, :, j, :] = e[:, :, 0, :]
    sel = select_blocks(p, k_mean, q=q)
    O, LSE = sparse_attention(p, q, k, v, sel["lists"])
    return O, LSE, sel["lists"]
