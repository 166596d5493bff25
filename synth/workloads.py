"""Seeded synthetic workloads shaped like the settings the pages describe.

No dataset, checkpoint or benchmark item is used or reproduced: every tensor is
drawn from a seeded generator and given planted structure of the kind the
pages talk about (retrievable "needle" blocks, topic blocks, a local window),
so that block selection and threshold skipping have something real to find.

Recipe shared by every workload
-------------------------------
* Each (tensor, head) pair draws from its own PCG64 stream seeded with
  ``SeedSequence([seed, tensor_code, head])``; any subset of heads can be
  regenerated alone, and the draw order inside one stream is fixed.
* Base values are N(0, 1) drawn in float32.  RoPE (when the workload uses it)
  is applied in float64 with base 10000; planted structure is added after RoPE
  so it stays visible at every distance.
* Values are rounded once at the end: float64 -> float32 (round to nearest
  even) -> bfloat16 (round to nearest even).  bf16 tensors are stored as their
  raw uint16 bit patterns.  The oracle reads exactly these stored values.
* Layout is [B, H, L, D] with the last dimension contiguous (B = 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ROPE_HALF = 0          # FC i pairs dims (i, i + D/2)
ROPE_INTERLEAVED = 1   # FC i pairs dims (2i, 2i + 1)
ROPE_BASE = 10000.0

# tensor codes for the per-(tensor, head) seed streams
_Q, _K, _V = 1, 2, 3


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


# ---------------------------------------------------------------- rounding ---
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x64, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


# -------------------------------------------------------------------- RoPE ---
def rope(x: np.ndarray, pos: np.ndarray, layout: int = ROPE_HALF, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate x[..., L, D] by RoPE at absolute positions pos[L] (float64).

    Frequency chunk i in [0, D/2) turns at theta_i = base^(-2i/D); low FC index
    means fast rotation.  This is data preparation: the library consumes
    already-rotated vectors and never applies RoPE itself.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    if layout == ROPE_HALF:
        a, b = x[..., :half], x[..., half:]
        out[..., :half] = a * c - b * s
        out[..., half:] = b * c + a * s
    elif layout == ROPE_INTERLEAVED:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
    else:
        raise ValueError(layout)
    return out


def hi_band_dims(D: int, layout: int) -> np.ndarray:
    """Dims of the fast-rotating half of the frequency chunks (FC i < D/4)."""
    fc = np.arange(D // 4)
    if layout == ROPE_HALF:
        return np.concatenate([fc, fc + D // 2])
    return np.stack([2 * fc, 2 * fc + 1], axis=1).reshape(-1)


def lo_band_dims(D: int, layout: int) -> np.ndarray:
    return np.setdiff1d(np.arange(D), hi_band_dims(D, layout))


def _normal(seed: int, code: int, head: int, shape) -> np.ndarray:
    return _rng(seed, code, head).standard_normal(shape, dtype=np.float32).astype(np.float64)


def _unit(rng: np.random.Generator, n: int, D: int, dims: np.ndarray | None = None) -> np.ndarray:
    v = np.zeros((n, D))
    d = np.arange(D) if dims is None else dims
    w = rng.standard_normal((n, len(d)))
    v[:, d] = w / np.linalg.norm(w, axis=1, keepdims=True)
    return v


# --------------------------------------------------------------- workload ---
@dataclass
class Workload:
    name: str
    dtype: str            # storage dtype of q, k, v: "bf16" (uint16 bits) or "f32"
    q: np.ndarray         # [1, Hq, Lq, D]
    k: np.ndarray         # [1, Hkv, L, D]
    v: np.ndarray         # [1, Hkv, L, D]
    params: dict          # method parameters (block sizes, budgets, flags)
    extra: dict = field(default_factory=dict)

    @property
    def shape(self):
        _, Hq, Lq, D = self.q.shape
        return dict(Hq=Hq, Hkv=self.k.shape[1], Lq=Lq, L=self.k.shape[2], D=D)

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name) if hasattr(self, name) else self.extra[name]
        return storage_to_f64(a, self.dtype)


def tiny_decode(seed: int = 1, L: int = 1024, D: int = 64, block: int = 64) -> Workload:
    """One query, one head, fp32, RoPE'd keys at 0..L-1 and the query at L-1.

    Budget of 4 blocks: block 0 and the newest block are forced, two more are
    scored picks (an NSA-style budget that counts its forced blocks).
    """
    pos_k = np.arange(L)
    q = rope(_normal(seed, _Q, 0, (1, D)), np.array([L - 1]))
    k = rope(_normal(seed, _K, 0, (L, D)), pos_k)
    v = _normal(seed, _V, 0, (L, D))
    params = dict(kv_block=block, q_block=1, q_pos0=L - 1, causal=0, topk=2, topk_num=0, topk_den=1,
                  n_first=1, n_last=1, dual_band=0, layout=ROPE_HALF, scale=1.0 / math.sqrt(D))
    return Workload("tiny_decode", "f32", _store(q[None, None], "f32"), _store(k[None, None], "f32"),
                    _store(v[None, None], "f32"), params)


def gqa_decode(seed: int = 2, L: int = 65536, Hq: int = 32, Hkv: int = 8, D: int = 128, block: int = 64,
               n_needles: int = 8) -> Workload:
    """GQA decode step over a long RoPE'd prefix, with planted needle blocks.

    Per KV head, ``n_needles`` blocks drawn from {1 .. NB-3} get keys
    0.5 * (mean of the group's RoPE'd queries) + N(0, 1).  Budget: 16 blocks =
    block 0 + the 2 newest + 13 scored picks (NSA's selection setting).
    """
    G = Hq // Hkv
    NB = -(-L // block)
    qpos = np.array([L - 1])
    q = np.stack([rope(_normal(seed, _Q, h, (1, D)), qpos) for h in range(Hq)])          # [Hq,1,D]
    kb = np.empty((Hkv, L, D), dtype=np.uint16)
    vb = np.empty((Hkv, L, D), dtype=np.uint16)
    needles = np.zeros((Hkv, n_needles), dtype=np.int64)
    pos_k = np.arange(L)
    for g in range(Hkv):
        kg = rope(_normal(seed, _K, g, (L, D)), pos_k)
        qbar = q[g * G:(g + 1) * G, 0].mean(axis=0)
        nd = np.sort(_rng(seed, 20, g).choice(np.arange(1, max(NB - 2, 2)), size=n_needles, replace=False))
        needles[g] = nd
        for j in nd:
            kg[j * block:min((j + 1) * block, L)] += 0.5 * qbar
        kb[g] = _store(kg, "bf16")
        vb[g] = _store(_normal(seed, _V, g, (L, D)), "bf16")
    params = dict(kv_block=block, q_block=1, q_pos0=L - 1, causal=0, topk=13, topk_num=0, topk_den=1,
                  n_first=1, n_last=2, dual_band=0, layout=ROPE_HALF, scale=1.0 / math.sqrt(D))
    return Workload("gqa_decode", "bf16", _store(q, "bf16")[None], kb[None], vb[None], params,
                    dict(needles=needles))


def dlm_denoise(seed: int = 3, L: int = 32768, R: int = 32, Hq: int = 32, Hkv: int = 8, D: int = 128,
                block: int = 64, n_active: int = 8, n_needles: int = 8, theta: float = 0.1) -> Workload:
    """One denoising step of a block-wise diffusion LM over a cached prefix.

    The query block has R rows at positions L .. L+R-1.  Previous-step queries
    (pre-RoPE) are u_g + N(0, 1) with a shared per-group direction u_g.  A
    seeded set of ``n_active`` rows changes by N(0, 1) (all heads); the other
    rows change by N(0, 0.01^2).  Per KV head, ``n_needles`` blocks get keys
    0.5 * (mean RoPE'd previous query of the group) + N(0, 1).
    Budget: 16 scored picks per row, no forced blocks, union over the block.
    """
    G = Hq // Hkv
    NB = -(-L // block)
    rpos = L + np.arange(R)
    u = np.stack([_rng(seed, 30, g).standard_normal(D) for g in range(Hkv)])
    q_prev = np.stack([rope(u[h // G][None, :] + _normal(seed, _Q, h, (R, D)), rpos) for h in range(Hq)])
    active = np.sort(_rng(seed, 31).choice(R, size=n_active, replace=False))
    is_act = np.zeros(R, dtype=bool)
    is_act[active] = True
    q_cur = np.empty_like(q_prev)
    for h in range(Hq):
        d = _rng(seed, 33, h).standard_normal((R, D))
        q_cur[h] = q_prev[h] + np.where(is_act[:, None], d, 0.01 * d)
    kb = np.empty((Hkv, L, D), dtype=np.uint16)
    vb = np.empty((Hkv, L, D), dtype=np.uint16)
    needles = np.zeros((Hkv, n_needles), dtype=np.int64)
    pos_k = np.arange(L)
    for g in range(Hkv):
        kg = rope(_normal(seed, _K, g, (L, D)), pos_k)
        qbar = q_prev[g * G:(g + 1) * G].reshape(-1, D).mean(axis=0)
        nd = np.sort(_rng(seed, 32, g).choice(NB, size=min(n_needles, NB), replace=False))
        needles[g, :len(nd)] = nd
        for j in nd:
            kg[j * block:min((j + 1) * block, L)] += 0.5 * qbar
        kb[g] = _store(kg, "bf16")
        vb[g] = _store(_normal(seed, _V, g, (L, D)), "bf16")
    params = dict(kv_block=block, q_block=R, q_pos0=L, causal=0, topk=16, topk_num=0, topk_den=1,
                  n_first=0, n_last=0, dual_band=0, layout=ROPE_HALF, scale=1.0 / math.sqrt(D),
                  theta_act=theta)
    return Workload("dlm_denoise", "bf16", _store(q_cur, "bf16")[None], kb[None], vb[None], params,
                    dict(q_prev=_store(q_prev, "bf16")[None], active=active, needles=needles))


def dlm_denoise_steps(seed: int = 6, L: int = 32768, R: int = 32, Hq: int = 32, Hkv: int = 8, D: int = 128,
                      block: int = 64, n_steps: int = 8, per_step: int = 4, n_needles: int = 8,
                      theta: float = 0.1) -> Workload:
    """Several denoising steps of one 32-token block over a cached prefix.

    The prefix K/V, needles and step-0 queries come from ``dlm_denoise`` (its
    previous-step queries are the queries of step 0).  The block's own keys
    and values sit at positions L .. L+R-1: step 0 draws RoPE'd N(0, 1) keys and
    N(0, 1) values.  At each later step ``per_step`` seeded rows that have not
    changed before are unmasked: their query vectors (all heads) change by
    N(0, 1) and their block keys/values are drawn afresh; every other row
    drifts by N(0, 0.01^2).  extra holds per-step lists ``q_steps``
    [1, Hq, R, D], ``kb_steps``/``vb_steps`` [1, Hkv, R, D] (bf16 bits) and the
    unmasked rows ``changed`` of each step (empty at step 0).
    """
    base = dlm_denoise(seed=seed, L=L, R=R, Hq=Hq, Hkv=Hkv, D=D, block=block, n_active=per_step,
                       n_needles=n_needles, theta=theta)
    rpos = L + np.arange(R)
    q = storage_to_f64(base.extra["q_prev"], "bf16")[0]
    kb = np.stack([rope(_rng(seed, 70, g).standard_normal((R, D)), rpos) for g in range(Hkv)])
    vb = np.stack([_rng(seed, 71, g).standard_normal((R, D)) for g in range(Hkv)])
    q_steps, kb_steps, vb_steps, changed = [_store(q, "bf16")[None]], [_store(kb, "bf16")[None]], \
        [_store(vb, "bf16")[None]], [np.zeros(0, dtype=np.int64)]
    fresh = np.ones(R, dtype=bool)
    for s in range(1, n_steps):
        cand = np.nonzero(fresh)[0]
        rows = np.sort(_rng(seed, 72, s).choice(cand, size=min(per_step, len(cand)), replace=False))
        fresh[rows] = False
        act = np.zeros(R, dtype=bool)
        act[rows] = True
        for h in range(Hq):
            d = _rng(seed, 73, s, h).standard_normal((R, D))
            q[h] = q[h] + np.where(act[:, None], d, 0.01 * d)
        for g in range(Hkv):
            nk = rope(_rng(seed, 74, s, g).standard_normal((R, D)), rpos)
            nv = _rng(seed, 75, s, g).standard_normal((R, D))
            kb[g] = np.where(act[:, None], nk, kb[g] + 0.01 * nk)
            vb[g] = np.where(act[:, None], nv, vb[g] + 0.01 * nv)
        q_steps.append(_store(q, "bf16")[None])
        kb_steps.append(_store(kb, "bf16")[None])
        vb_steps.append(_store(vb, "bf16")[None])
        changed.append(rows.astype(np.int64))
    extra = dict(base.extra, q_steps=q_steps, kb_steps=kb_steps, vb_steps=vb_steps, changed=changed)
    return Workload("dlm_denoise_steps", "bf16", q_steps[0], base.k, base.v, dict(base.params), extra)


def sparse_prefill(seed: int = 4, L: int = 32768, Hq: int = 32, Hkv: int = 8, D: int = 128, block: int = 128,
                   n_topics: int = 16, topic_frac: float = 0.25, amp: float = 4.0, c_norm2: float = 64.0) -> Workload:
    """Causal prefill with both a positional (fast band) and a topical (slow band) signal.

    Interleaved RoPE layout, so the fast-rotating chunks are literally the
    lower half of the head dims and the slow ones the upper half.
    (i)  a fixed per-group vector c_g on fast-band dims, |c_g|^2 = c_norm2, is
         added to every pre-RoPE query and key of the group: after RoPE it
         yields a local ("slash") preference;
    (ii) ``n_topics`` unit topic vectors per group on slow-band dims; every
         query block and ``topic_frac`` of the key blocks get one topic,
         amplitude ``amp``, added after RoPE.
    Budget per query block i: blocks {0, i} plus ceil(0.10 * (i + 1)) scored picks.
    """
    G = Hq // Hkv
    NB = -(-L // block)
    layout = ROPE_INTERLEAVED
    hi = hi_band_dims(D, layout)
    lo = lo_band_dims(D, layout)
    pos = np.arange(L)
    qb = np.empty((Hq, L, D), dtype=np.uint16)
    kb = np.empty((Hkv, L, D), dtype=np.uint16)
    vb = np.empty((Hkv, L, D), dtype=np.uint16)
    q_topic = np.zeros((Hkv, NB), dtype=np.int64)
    k_topic = np.full((Hkv, NB), -1, dtype=np.int64)
    for g in range(Hkv):
        c = _unit(_rng(seed, 40, g), 1, D, hi)[0] * math.sqrt(c_norm2)
        topics = _unit(_rng(seed, 41, g), n_topics, D, lo)
        qt = _rng(seed, 42, g).integers(0, n_topics, size=NB)
        rk = _rng(seed, 43, g)
        kblocks = np.sort(rk.choice(NB, size=int(round(topic_frac * NB)), replace=False))
        kt = rk.integers(0, n_topics, size=len(kblocks))
        q_topic[g] = qt
        k_topic[g, kblocks] = kt
        qadd = np.repeat(amp * topics[qt], block, axis=0)[:L]
        for h in range(g * G, (g + 1) * G):
            qh = rope(_normal(seed, _Q, h, (L, D)) + c, pos, layout) + qadd
            qb[h] = _store(qh, "bf16")
        kg = rope(_normal(seed, _K, g, (L, D)) + c, pos, layout)
        for j, t in zip(kblocks, kt):
            kg[j * block:min((j + 1) * block, L)] += amp * topics[t]
        kb[g] = _store(kg, "bf16")
        vb[g] = _store(_normal(seed, _V, g, (L, D)), "bf16")
    params = dict(kv_block=block, q_block=block, q_pos0=0, causal=1, topk=0, topk_num=1, topk_den=10,
                  n_first=1, n_last=1, dual_band=1, layout=layout, scale=1.0 / math.sqrt(D))
    return Workload("sparse_prefill", "bf16", qb[None], kb[None], vb[None], params,
                    dict(q_topic=q_topic, k_topic=k_topic))


def threshold_prefill(seed: int = 5, L: int = 131072, Hq: int = 32, Hkv: int = 8, D: int = 128, tile: int = 128,
                      seg_tiles: int = 108, n_needles: int = 8, lam: float = 1e-3, logit_gap: float = 24.0,
                      heads: list[int] | None = None) -> Workload:
    """Causal prefill without RoPE, for the softmax-threshold skip.

    Tokens fall into segments of ``seg_tiles`` tiles, each with a random unit
    code e_m per group.  Queries add alpha*e_seg(r); keys add
    alpha*(e_seg(s) + e_seg(s)+1), so a query sees its own and the previous
    segment strongly (a local window).  Per KV head, ``n_needles`` tiles carry
    alpha*w_g in their keys instead of the segment codes, while every query of
    the group adds alpha*w_g: a needle is seen by every later query.
    alpha^2 / sqrt(D) = ``logit_gap``.  Everything outside the window and the
    needles sits far below the running max, so about 70% of causal tiles are
    skippable at lambda = 1e-3 with the default sizes.

    ``heads`` limits generation to some query heads (their KV heads are made
    in full); other heads are left zero.  Used to bound host time when only a
    sample of heads is checked.
    """
    G = Hq // Hkv
    NT = -(-L // tile)
    nseg = -(-NT // seg_tiles) + 1
    alpha = math.sqrt(logit_gap * math.sqrt(D))
    seg = (np.arange(L) // tile) // seg_tiles
    qb = np.zeros((Hq, L, D), dtype=np.uint16)
    kb = np.zeros((Hkv, L, D), dtype=np.uint16)
    vb = np.zeros((Hkv, L, D), dtype=np.uint16)
    needles = np.zeros((Hkv, n_needles), dtype=np.int64)
    want = set(range(Hq)) if heads is None else set(heads)
    for g in range(Hkv):
        hs = [h for h in range(g * G, (g + 1) * G) if h in want]
        if not hs:
            continue
        e = _unit(_rng(seed, 50, g), nseg + 1, D)
        nd = np.sort(_rng(seed, 51, g).choice(NT, size=min(n_needles, NT), replace=False))
        w = _unit(_rng(seed, 52, g), 1, D)[0]
        needles[g, :len(nd)] = nd
        qstruct = alpha * (e[seg] + w[None, :])
        for h in hs:
            qb[h] = _store(_normal(seed, _Q, h, (L, D)) + qstruct, "bf16")
        kstruct = alpha * (e[seg] + e[seg + 1])
        for t in nd:
            # a needle tile carries the needle code instead of its segment codes, so
            # inside a query's window it scores like the window, not twice as high
            kstruct[t * tile:min((t + 1) * tile, L)] = alpha * w
        kg = _normal(seed, _K, g, (L, D)) + kstruct
        kb[g] = _store(kg, "bf16")
        vb[g] = _store(_normal(seed, _V, g, (L, D)), "bf16")
    params = dict(tile=tile, causal=1, lam=lam, scale=1.0 / math.sqrt(D))
    return Workload("threshold_prefill", "bf16", qb[None], kb[None], vb[None], params,
                    dict(needles=needles, seg_tiles=seg_tiles, alpha=alpha))


def threshold_decode(seed: int = 5, L: int = 65536, Hq: int = 32, Hkv: int = 8, D: int = 128, tile: int = 128,
                     seg_tiles: int = 108, n_needles: int = 8, logit_gap: float = 24.0) -> Workload:
    """One decode query per head over a cache with the threshold-prefill
    structure (local segments and needles, no RoPE): the query, at position
    L - 1, carries alpha*(e_seg(L-1) + w_g), so it sees its own and the
    previous segment and the needles; the rest of the cache sits far below the
    running max.  K and V are made exactly as threshold_prefill makes them; the
    query's noise comes from its own stream."""
    G = Hq // Hkv
    NT = -(-L // tile)
    nseg = -(-NT // seg_tiles) + 1
    alpha = math.sqrt(logit_gap * math.sqrt(D))
    seg = (np.arange(L) // tile) // seg_tiles
    qb = np.zeros((Hq, 1, D), dtype=np.uint16)
    kb = np.zeros((Hkv, L, D), dtype=np.uint16)
    vb = np.zeros((Hkv, L, D), dtype=np.uint16)
    needles = np.zeros((Hkv, n_needles), dtype=np.int64)
    for g in range(Hkv):
        e = _unit(_rng(seed, 50, g), nseg + 1, D)
        nd = np.sort(_rng(seed, 51, g).choice(NT, size=min(n_needles, NT), replace=False))
        w = _unit(_rng(seed, 52, g), 1, D)[0]
        needles[g, :len(nd)] = nd
        for h in range(g * G, (g + 1) * G):
            qb[h] = _store(_normal(seed, _Q + 100, h, (1, D)) + alpha * (e[seg[L - 1]] + w)[None, :], "bf16")
        kstruct = alpha * (e[seg] + e[seg + 1])
        for t in nd:
            kstruct[t * tile:min((t + 1) * tile, L)] = alpha * w
        kb[g] = _store(_normal(seed, _K, g, (L, D)) + kstruct, "bf16")
        vb[g] = _store(_normal(seed, _V, g, (L, D)), "bf16")
    params = dict(q_pos0=L - 1, causal=1, scale=1.0 / math.sqrt(D))
    return Workload("threshold_decode", "bf16", qb[None], kb[None], vb[None], params,
                    dict(needles=needles, seg_tiles=seg_tiles, alpha=alpha))


def decode_batch_shifts(B: int, L: int, block: int, seed: int = 11) -> list:
    """Token shifts that turn one GQA decode cache into a batch of B distinct
    sequences: sequence b holds the base cache circularly shifted by
    shifts[b] tokens along L (np.roll semantics, a multiple of the block size,
    so blocks stay whole and the planted needles move to other blocks).
    shifts[0] = 0 and the shifts are distinct, so every sequence selects its
    own blocks; the query rows are the base workload's for every sequence."""
    NB = -(-L // block)
    if L % block:
        raise ValueError("the batch shifts need L to be a multiple of the block size")
    if B > NB:
        raise ValueError("more sequences than blocks")
    rest = _rng(seed, 70).permutation(np.arange(1, NB))[:B - 1]
    return [0] + [int(j) * block for j in rest]


def shift_sequence(x: np.ndarray, shift: int) -> np.ndarray:
    """One sequence of a shifted batch: x [H, L, D] rolled by `shift` tokens."""
    return np.roll(x, shift, axis=1)


def decode_rows(seed: int = 7, Lq: int = 128, L: int = 4096, Hq: int = 32, Hkv: int = 8, D: int = 128,
                block: int = 64, cap: int = 16) -> Workload:
    """Many single-row query blocks at once (rows decoded together over one
    shared prefix), each with its own given block list: per (KV head, row) a
    count drawn uniformly from 0 .. cap (every seventh row of KV head 0 gets an
    empty list), the blocks drawn without replacement from the NB blocks and
    sorted.  No RoPE; N(0, 1) queries, keys and values.  extra: idx
    [1, Hkv, Lq, cap] int32 (-1 past the count), cnt [1, Hkv, Lq] int32."""
    NB = -(-L // block)
    qb = np.stack([_store(_normal(seed, _Q, h, (Lq, D)), "bf16") for h in range(Hq)])
    kb = np.stack([_store(_normal(seed, _K, g, (L, D)), "bf16") for g in range(Hkv)])
    vb = np.stack([_store(_normal(seed, _V, g, (L, D)), "bf16") for g in range(Hkv)])
    idx = np.full((1, Hkv, Lq, cap), -1, dtype=np.int32)
    cnt = np.zeros((1, Hkv, Lq), dtype=np.int32)
    for g in range(Hkv):
        rng = _rng(seed, 60, g)
        for r in range(Lq):
            n = 0 if (g == 0 and r % 7 == 0) else int(rng.integers(0, min(cap, NB) + 1))
            cnt[0, g, r] = n
            idx[0, g, r, :n] = np.sort(rng.choice(NB, size=n, replace=False))
    params = dict(kv_block=block, q_block=1, q_pos0=L - Lq, causal=0, cap=cap, scale=1.0 / math.sqrt(D))
    return Workload("decode_rows", "bf16", qb[None], kb[None], vb[None], params, dict(idx=idx, cnt=cnt))
