"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against mathematics the pages imply, a library
routine on a special case, brute force on tiny inputs, or structure planted by
the seeded generators -- never against a retyped copy of its own formula.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle as orc
import synth
from synth.workloads import ROPE_HALF, ROPE_INTERLEAVED

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = float(v)
    return out


def _dense(q, k, v, scale, qpos=None):
    """Plain dense attention by library softmax/logsumexp (independent path)."""
    S = scale * np.einsum("rd,td->rt", q, k)
    if qpos is not None:
        S = np.where(np.arange(k.shape[0])[None, :] <= qpos[:, None], S, -np.inf)
    return softmax(S, axis=1) @ v, logsumexp(S, axis=1)


def _fc_pairs(D, layout):
    i = np.arange(D // 2)
    return (i, i + D // 2) if layout == ROPE_HALF else (2 * i, 2 * i + 1)


# ------------------------------------------------------------- bands / RoPE ---
@pytest.mark.parametrize("layout", [ROPE_HALF, ROPE_INTERLEAVED])
def test_band_energy_is_rotation_invariant(layout):
    """RoPE turns each frequency chunk rigidly, so a band made of whole chunks keeps
    its energy at every position.  A band mask that split a chunk would not."""
    D, L = 32, 96
    rng = np.random.default_rng(0)
    c = rng.standard_normal(D)
    x = synth.rope(np.tile(c, (L, 1)), np.arange(L) * 7 + 3, layout)
    _, e = orc.block_summaries(x[None], 1, layout)
    fast = orc.fast_band_mask(D, layout)
    assert np.allclose(e[0, :, 0], np.sum(c[fast] ** 2), rtol=1e-12)
    assert np.allclose(e[0, :, 1], np.sum(c[~fast] ** 2), rtol=1e-12)
    # the fast band is FC index < D/4 (high frequency = low FC index)
    a, b = _fc_pairs(D, layout)
    assert fast[a[: D // 4]].all() and fast[b[: D // 4]].all()
    assert not fast[a[D // 4:]].any() and not fast[b[D // 4:]].any()


@pytest.mark.parametrize("layout", [ROPE_HALF, ROPE_INTERLEAVED])
@pytest.mark.parametrize("block", [64, 128])
def test_pooling_is_dirichlet_low_pass(layout, block):
    """Mean pooling of a RoPE'd constant vector: chunk i keeps amplitude
    |c_i| * |sin(b*theta_i/2) / (b*sin(theta_i/2))| (geometric-sum identity), for
    any start position -- the low-pass claim of the Prism page made exact."""
    D, base = 128, 10000.0
    rng = np.random.default_rng(1)
    c = rng.standard_normal(D)
    p0 = 37 * block + 5
    x = synth.rope(np.tile(c, (block, 1)), p0 + np.arange(block), layout)
    mean, energy = orc.block_summaries(x[None], block, layout)
    a, b = _fc_pairs(D, layout)
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    dk = np.abs(np.sin(block * theta / 2) / (block * np.sin(theta / 2)))
    amp_in = np.hypot(c[a], c[b])
    amp_out = np.hypot(mean[0, 0, a], mean[0, 0, b])
    assert np.allclose(amp_out, amp_in * dk, rtol=1e-9, atol=1e-12)
    # retained fraction per band follows from the same identity
    fast = orc.fast_band_mask(D, layout)
    rho = orc.retained_fraction(mean[None], energy[None], layout)[0, 0]
    fc_fast = np.arange(D // 2) < D // 4
    exp_fast = np.sum((amp_in * dk)[fc_fast] ** 2) / np.sum(c[fast] ** 2)
    exp_slow = np.sum((amp_in * dk)[~fc_fast] ** 2) / np.sum(c[~fast] ** 2)
    assert np.allclose(rho, [exp_fast, exp_slow], rtol=1e-9)


def test_dirichlet_spot_values():
    """A few values of the squared pooling gain (base 1e4, D = 128)."""
    theta = lambda i: 10000.0 ** (-2.0 * i / 128)
    gain2 = lambda b, i: (math.sin(b * theta(i) / 2) / (b * math.sin(theta(i) / 2))) ** 2
    assert gain2(64, 0) == pytest.approx(3.23e-4, rel=2e-2)
    assert gain2(64, 31) == pytest.approx(0.955, abs=1e-3)
    assert gain2(128, 24) == pytest.approx(0.197, abs=2e-3)
    assert gain2(128, 32) == pytest.approx(0.871, abs=1e-3)


# ---------------------------------------------------------------- summaries ---
def test_summaries_ragged_last_block():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 150, 16))
    mean, energy = orc.block_summaries(x, 64, ROPE_HALF)
    assert mean.shape == (2, 3, 3, 16)
    assert np.allclose(mean[..., 2, :], np.mean(x[..., 128:, :], axis=-2))
    assert np.allclose(energy.sum(-1)[..., 2], np.mean(np.sum(x[..., 128:, :] ** 2, -1), -1))


# ------------------------------------------------------------- temperatures ---
def test_temperature_invariances():
    rng = np.random.default_rng(3)
    D, G = 32, 2
    k = rng.standard_normal((1, 2, 2048, D))
    q = rng.standard_normal((1, 4, 2048, D))
    km, ke = orc.block_summaries(k, 32, ROPE_HALF)
    qm, qe = orc.block_summaries(q, 32, ROPE_HALF)
    t1 = orc.band_temperatures(km, ke, ROPE_HALF, G, qm, qe)
    km2, ke2 = orc.block_summaries(3.7 * k, 32, ROPE_HALF)
    assert np.allclose(orc.band_temperatures(km2, ke2, ROPE_HALF, G, qm, qe), t1, rtol=1e-12)
    # no variation inside blocks -> pooling keeps everything -> tau = 1
    kc = np.repeat(rng.standard_normal((1, 2, 8, D)), 32, axis=2)
    kmc, kec = orc.block_summaries(kc, 32, ROPE_HALF)
    assert np.allclose(orc.band_temperatures(kmc, kec, ROPE_HALF, G), 1.0, rtol=1e-12)
    # i.i.d. noise: pooling 32 tokens keeps about 1/32 of the energy -> tau ~ 1/32
    assert np.allclose(t1, 1.0 / 32, rtol=0.15)


# ------------------------------------------------------------------ scoring ---
def test_single_head_ranking_is_dot_product_order():
    """G = 1, one band: softmax is monotone, so the ranking is argsort(q . kbar)."""
    rng = np.random.default_rng(4)
    qr = rng.standard_normal((1, 16))
    km = rng.standard_normal((40, 16))
    s = orc.group_scores(qr, km, 0.25)
    assert np.array_equal(np.argsort(-s, kind="stable"), np.argsort(-(km @ qr[0]), kind="stable"))
    assert s.sum() == pytest.approx(1.0)


def test_group_score_is_sum_of_head_probabilities():
    rng = np.random.default_rng(5)
    qr = rng.standard_normal((4, 16))
    km = rng.standard_normal((30, 16))
    s = orc.group_scores(qr, km, 0.3)
    assert s.sum() == pytest.approx(4.0)
    assert np.allclose(s, sum(softmax(0.3 * km @ qr[h]) for h in range(4)))


def test_dual_band_reduces_to_slow_band_when_fast_band_is_empty():
    """With zero fast-band components the fast softmax is uniform, so the
    ranking is argsort of the slow-band dot product."""
    rng = np.random.default_rng(6)
    D = 32
    fast = orc.fast_band_mask(D, ROPE_INTERLEAVED)
    qr = rng.standard_normal((1, D))
    km = rng.standard_normal((25, D))
    qr[:, fast] = 0
    km[:, fast] = 0
    tau = np.array([[0.3, 0.7]])
    s = orc.group_scores(qr, km, 0.2, tau, fast)
    assert np.allclose(s, 0.5 / 25 + 0.5 * softmax(0.2 * (km @ qr[0]) / 0.7))
    assert np.array_equal(np.argsort(-s, kind="stable"), np.argsort(-(km @ qr[0]), kind="stable"))


# ---------------------------------------------------------------- selection ---
def test_topk_brute_force_tiny():
    """Every k'-subset enumerated: the oracle's picks maximise the summed group
    score (ties -> lexicographically smaller indices)."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        NB, D, G = int(rng.integers(3, 9)), 8, int(rng.integers(1, 3))
        qr = rng.standard_normal((G, D))
        km = rng.standard_normal((NB, D))
        if trial % 5 == 0:
            km[1] = km[3 % NB]          # exact ties
        C = np.arange(NB)
        F = orc.forced_blocks(C, dict(n_first=1, n_last=1))
        kp = int(rng.integers(0, NB - len(F) + 1))
        s = orc.group_scores(qr, km, 0.35)
        picks, _ = orc.top_picks(s, C, F, kp)
        free = [j for j in C if j not in F]
        best = max(itertools.combinations(free, kp), key=lambda S: (round(sum(s[list(S)]), 12), [-j for j in S]))
        assert np.array_equal(picks, np.array(sorted(set(F) | set(best))))


def test_nsa_budget_counts():
    """Decode budget: exactly 16 blocks of 64 = block 0 + the 2 newest + 13 picks."""
    g = _golden("nsa_selection.txt")
    w = synth.gqa_decode(L=8192, Hq=8, Hkv=2)
    p = w.params
    assert p["kv_block"] == g["selection_block"]
    assert p["n_first"] == g["initial_blocks"] and p["n_last"] == g["local_blocks"]
    assert p["topk"] + p["n_first"] + p["n_last"] == g["selected_blocks"]
    q, k = w.f64("q"), w.f64("k")
    km, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    sel = orc.select_blocks(p, km, q=q)
    NB = km.shape[2]
    for g_ in range(2):
        lst = sel["lists"][0][g_][0]
        assert len(lst) == 16 and len(np.unique(lst)) == 16
        assert {0, NB - 2, NB - 1} <= set(lst.tolist())
        # planted needles (keys = 0.5 * mean query + noise) are all found
        assert set(w.extra["needles"][g_].tolist()) <= set(lst.tolist())


def test_prefill_budget_count_formula():
    """Causal prefill lists: {0, i} + ceil((i+1)/10) picks, capped by the candidates."""
    p = dict(kv_block=128, q_block=128, q_pos0=0, causal=1, topk=0, topk_num=1, topk_den=10,
             n_first=1, n_last=1)

    def size(i):
        C = orc.candidate_blocks(i, 10**6, p, 10**9)
        F = orc.forced_blocks(C, p)
        return len(F) + orc.num_scored_picks(len(C), len(F), p)

    expect = lambda i: min(i + 1, (2 if i else 1) + (i + 10) // 10)
    assert all(size(i) == expect(i) for i in range(400))
    assert sum(expect(i) for i in range(256)) == 3915


def test_union_properties_and_active_subset():
    w = synth.dlm_denoise(L=2048, R=16, Hq=4, Hkv=2, n_active=4, n_needles=2)
    p = w.params
    q, k = w.f64("q"), w.f64("k")
    km, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    mask, mse = orc.active_rows(q, w.f64("q_prev"), p["theta_act"])
    # the generator planted exactly these active rows (change N(0,1) vs N(0,1e-4))
    assert np.array_equal(np.nonzero(mask[0])[0], w.extra["active"])
    s_all = orc.select_blocks(p, km, q=q)
    s_act = orc.select_blocks(p, km, q=q, row_mask=mask)
    for g in range(2):
        U = s_all["lists"][0][g][0]
        picks = [s_all["rows"][(0, g, r)]["picks"] for r in range(16)]
        assert np.array_equal(U, np.array(sorted(set(np.concatenate(picks).tolist()))))
        assert len(U) == len(set(np.concatenate(picks).tolist()))
        assert all(len(pk) == 16 and set(pk.tolist()) <= set(U.tolist()) for pk in picks)
        Ua = s_act["lists"][0][g][0]
        assert set(Ua.tolist()) <= set(U.tolist()) and len(Ua) < len(U)


# ---------------------------------------------------------------- attention ---
def test_select_everything_equals_dense_decode():
    rng = np.random.default_rng(8)
    L, D = 300, 16
    q = rng.standard_normal((1, 4, 1, D))
    k = rng.standard_normal((1, 2, L, D))
    v = rng.standard_normal((1, 2, L, D))
    p = dict(kv_block=32, q_block=1, q_pos0=L - 1, causal=0, topk=100, n_first=1, n_last=2, scale=0.25,
             layout=ROPE_HALF)
    km, _ = orc.block_summaries(k, 32, ROPE_HALF)
    sel = orc.select_blocks(p, km, q=q)
    O, lse = orc.sparse_attention(p, q, k, v, sel["lists"])
    for h in range(4):
        o2, l2 = _dense(q[0, h], k[0, h // 2], v[0, h // 2], 0.25)
        assert np.allclose(O[0, h], o2, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[0, h], l2, rtol=1e-12)


def test_select_everything_equals_dense_causal_prefill():
    rng = np.random.default_rng(9)
    L, D, b = 200, 16, 32      # ragged: 7 blocks, the last has 8 tokens
    q = rng.standard_normal((1, 2, L, D))
    k = rng.standard_normal((1, 1, L, D))
    v = rng.standard_normal((1, 1, L, D))
    p = dict(kv_block=b, q_block=b, q_pos0=0, causal=1, topk=0, topk_num=1, topk_den=1, n_first=1,
             n_last=1, dual_band=1, layout=ROPE_INTERLEAVED, scale=0.25)
    km, ke = orc.block_summaries(k, b, p["layout"])
    qm, qe = orc.block_summaries(q, b, p["layout"])
    tau = orc.band_temperatures(km, ke, p["layout"], 2, qm, qe)
    sel = orc.select_blocks(p, km, q_mean=qm, tau=tau, Lq=L)
    assert all(len(sel["lists"][0][0][i]) == i + 1 for i in range(7))
    O, lse = orc.sparse_attention(p, q, k, v, sel["lists"])
    for h in range(2):
        o2, l2 = _dense(q[0, h], k[0, 0], v[0, 0], 0.25, np.arange(L))
        assert np.allclose(O[0, h], o2, rtol=1e-11, atol=1e-12)
        assert np.allclose(lse[0, h], l2, rtol=1e-12)


def test_uniform_keys_closed_form():
    """All keys equal: uniform weights, O = mean(v), LSE = s + ln(n) (natural log)."""
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 8))
    kk = np.tile(rng.standard_normal(8), (50, 1))
    v = rng.standard_normal((50, 8))
    O, lse = orc.attend_tokens(q, kk, v, np.arange(50), 0.5)
    assert np.allclose(O, v.mean(0)[None], atol=1e-13)
    assert np.allclose(lse, 0.5 * q @ kk[0] + math.log(50))


def test_lse_merge_of_disjoint_halves():
    """Attention over U split in two disjoint halves and merged by (O, LSE) equals one pass."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((400, 16))
    v = rng.standard_normal((400, 16))
    toks = np.sort(rng.choice(400, 180, replace=False))
    O, lse = orc.attend_tokens(q, k, v, toks, 0.3)
    O1, l1 = orc.attend_tokens(q, k, v, toks[:77], 0.3)
    O2, l2 = orc.attend_tokens(q, k, v, toks[77:], 0.3)
    L = np.logaddexp(l1, l2)
    assert np.allclose(L, lse)
    assert np.allclose(np.exp(l1 - L)[:, None] * O1 + np.exp(l2 - L)[:, None] * O2, O)


def test_merge_states_is_softmax_over_the_union():
    """merge_states of the states over two disjoint key sets equals one pass over
    their union (scipy's logsumexp and softmax for the one pass), including an
    empty side (LSE -inf, garbage O) and both sides empty."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((6, 16))
    k = rng.standard_normal((300, 16))
    v = rng.standard_normal((300, 16))
    for na in (0, 1, 120, 300):
        perm = rng.permutation(300)
        A, Bs = np.sort(perm[:na]), np.sort(perm[na:])
        Oa, La = orc.attend_tokens(q, k, v, A, 0.4)
        Ob, Lb = orc.attend_tokens(q, k, v, Bs, 0.4)
        if na == 0:
            Oa = np.full_like(Oa, 7.0)                 # ignored: the set is empty
        if na == 300:
            Ob = np.full_like(Ob, np.nan)
        O, L = orc.merge_states(Oa, La, Ob, Lb)
        S = 0.4 * q @ k.T
        assert np.allclose(L, logsumexp(S, axis=1), atol=1e-12)
        assert np.allclose(O, softmax(S, axis=1) @ v, atol=1e-12)
    O, L = orc.merge_states(np.ones((2, 4)), np.full(2, -np.inf), np.ones((2, 4)), np.full(2, -np.inf))
    assert np.all(O == 0) and np.all(L == -np.inf)


def test_denoise_first_step_is_dense_over_prefix_and_block():
    """The dense first step (every prefix block listed, every row) plus the
    block's own keys is the full softmax over [prefix; block] (scipy)."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, R, D, L, blk = 1, 4, 2, 8, 16, 200, 64
    q = rng.standard_normal((B, Hq, R, D))
    k, v = rng.standard_normal((B, Hkv, L, D)), rng.standard_normal((B, Hkv, L, D))
    kb, vb = rng.standard_normal((B, Hkv, R, D)), rng.standard_normal((B, Hkv, R, D))
    p = dict(kv_block=blk, q_block=R, q_pos0=L, causal=0, scale=0.25)
    lists = [[[np.arange(-(-L // blk))] for _ in range(Hkv)]]
    cO, cL = np.zeros((B, Hq, R, D)), np.zeros((B, Hq, R))
    O, Lse, cO2, cL2 = orc.denoise_step(p, q, k, v, kb, vb, lists, None, cO, cL)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        kk, vv = np.concatenate([k[0, g], kb[0, g]]), np.concatenate([v[0, g], vb[0, g]])
        S = 0.25 * q[0, h] @ kk.T
        assert np.allclose(Lse[0, h], logsumexp(S, axis=1), atol=1e-12)
        assert np.allclose(O[0, h], softmax(S, axis=1) @ vv, atol=1e-12)
        Sp = 0.25 * q[0, h] @ k[0, g].T                # the cache holds the prefix part alone
        assert np.allclose(cL2[0, h], logsumexp(Sp, axis=1), atol=1e-12)
    # a later step where no row is active: the cache is kept as is, and each
    # row is its cached prefix state merged with the new block part
    kb2 = rng.standard_normal(kb.shape)
    O3, L3, cO3, cL3 = orc.denoise_step(p, q, k, v, kb2, vb, lists, np.zeros((B, R), dtype=bool), cO2, cL2)
    assert np.array_equal(cO3, cO2) and np.array_equal(cL3, cL2)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        S = 0.25 * q[0, h] @ np.concatenate([k[0, g], kb2[0, g]]).T
        assert np.allclose(L3[0, h], logsumexp(S, axis=1), atol=1e-12)


def test_window_decode_branches():
    """Selection + sliding window: the window branch is scipy's softmax over the
    w keys ending at the row (clipped at the start); with w = L and gates
    (0, 1) the result is dense attention; with gates (1, 0) it is the list
    branch alone."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, Lq, D, L, blk = 1, 4, 2, 3, 16, 300, 64
    q = rng.standard_normal((B, Hq, Lq, D))
    k, v = rng.standard_normal((B, Hkv, L, D)), rng.standard_normal((B, Hkv, L, D))
    p = dict(kv_block=blk, q_block=1, q_pos0=100, causal=1, scale=0.3)
    lists = [[[np.array([0, 1]), np.array([1]), np.array([0])] for _ in range(Hkv)]]
    gates = rng.uniform(0.2, 1.5, (B, Hq, Lq, 2))
    O, LSE = orc.window_decode(p, q, k, v, lists, 40, gates)
    O_sel, L_sel = orc.sparse_attention(p, q, k, v, lists)
    for h in range(Hq):
        g = h // 2
        for r in range(Lq):
            pos = 100 + r
            S = 0.3 * k[0, g, pos - 39:pos + 1] @ q[0, h, r]
            o_w = softmax(S) @ v[0, g, pos - 39:pos + 1]
            assert np.isclose(LSE[0, h, r, 1], logsumexp(S))
            assert np.allclose(O[0, h, r], gates[0, h, r, 0] * O_sel[0, h, r] + gates[0, h, r, 1] * o_w)
    # a window longer than the prefix before the row is clipped at key 0
    O2, L2 = orc.window_decode(p, q, k, v, lists, 5000, np.stack([np.zeros((B, Hq, Lq)), np.ones((B, Hq, Lq))], -1))
    for h in range(Hq):
        for r in range(Lq):
            S = 0.3 * k[0, h // 2, :101 + r] @ q[0, h, r]
            assert np.allclose(O2[0, h, r], softmax(S) @ v[0, h // 2, :101 + r])
    O3, _ = orc.window_decode(p, q, k, v, lists, 7, np.stack([np.ones((B, Hq, Lq)), np.zeros((B, Hq, Lq))], -1))
    assert np.allclose(O3, O_sel)


@pytest.mark.parametrize("layout", [ROPE_HALF, ROPE_INTERLEAVED])
def test_token_scores_follow_the_rope_chunks(layout):
    """Per-chunk scores add up to q . k, and one chunk's score depends only on
    the distance between the two positions once q and k are rotated with RoPE
    (synth.rope in the same layout): a wrong dim pairing breaks it."""
    rng = np.random.default_rng(15)
    D, L = 32, 40
    q0, k0 = rng.standard_normal((1, D)), rng.standard_normal((L, D))
    allm = np.ones((1, D // 2), dtype=np.uint8)
    q, k = q0[None, None], k0[None, None]
    full = orc.token_scores(q, k, allm, layout)
    assert np.allclose(full[0, 0], k0 @ q0[0])
    parts = sum(orc.token_scores(q, k, np.eye(D // 2, dtype=np.uint8)[[f]], layout) for f in range(D // 2))
    assert np.allclose(parts, full)
    for f in (0, 5, D // 2 - 1):
        m = np.eye(D // 2, dtype=np.uint8)[[f]]
        sc = []
        for shift in (0, 17, 300):
            qr = synth.rope(q0, np.array([50 + shift]), layout)
            kr = synth.rope(k0, np.arange(L) + shift, layout)
            sc.append(orc.token_scores(qr[None, None], kr[None, None], m, layout)[0, 0])
        assert np.allclose(sc[0], sc[1]) and np.allclose(sc[0], sc[2])


def test_top_tokens_brute_force_with_ties():
    rng = np.random.default_rng(16)
    s = rng.integers(0, 6, 50).astype(float)           # many ties
    for budget in (1, 7, 20, 50, 80):
        toks, kth = orc.top_tokens(s, budget)
        n = min(budget, 50)
        assert len(toks) == n and np.all(np.diff(toks) > 0)
        best = [t for _, t in sorted((-s[t], t) for t in range(50))][:n]
        assert set(best) == set(toks.tolist()) and kth == min(s[best])


def test_token_attention_with_every_token_is_dense():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((1, 4, 1, 16))
    k, v = rng.standard_normal((1, 2, 90, 16)), rng.standard_normal((1, 2, 90, 16))
    lists = [[np.arange(90) for _ in range(4)]]
    O, L = orc.token_attention(q, k, v, lists, 0.25)
    for h in range(4):
        S = 0.25 * k[0, h // 2] @ q[0, h, 0]
        assert np.allclose(O[0, h, 0], softmax(S) @ v[0, h // 2]) and np.isclose(L[0, h, 0], logsumexp(S))


def test_causal_row_with_no_visible_key():
    q = np.ones((1, 4))
    O, lse = orc.attend_tokens(q, np.ones((4, 4)), np.ones((4, 4)), np.arange(2, 4), 1.0, np.array([1]))
    assert np.all(O == 0) and lse[0] == -np.inf


# ------------------------------------------------------ threshold attention ---
def _hand_example():
    # one query row (position 7, non-causal view of 8 keys in tiles of 2), q = e1,
    # key logits per tile: t0 = [0, -3], t1 = [2, 1], t2 = [-9, -8], t3 = [5, 4]
    a = np.array([0.0, -3.0, 2.0, 1.0, -9.0, -8.0, 5.0, 4.0])
    q = np.zeros((1, 4)); q[0, 0] = 1.0
    k = np.zeros((8, 4)); k[:, 0] = a
    v = np.random.default_rng(12).standard_normal((8, 4))
    return q, k, v, a


@pytest.mark.parametrize("lam,kept", [
    # visit 3 (max 5, first: keep, m=5); 2 (-8-5=-13); 1 (2-5=-3); 0 (0-5=-5)
    (1e-3, [0, 1, 3]),    # ln = -6.91: skip only tile 2
    (0.1, [3]),           # ln = -2.30: skip 2, 1, 0
    (0.04, [1, 3]),       # ln = -3.22: keep 1 (-3), skip 0 (-5)
    (0.0, [0, 1, 2, 3]),  # ln = -inf: never skip
])
def test_threshold_hand_example(lam, kept):
    q, k, v, a = _hand_example()
    r = orc.threshold_walk(q, k, v, np.array([7]), 2, lam, 1.0, causal=False)
    assert r["kept"] == kept
    toks = np.concatenate([[2 * j, 2 * j + 1] for j in kept])
    w = softmax(a[toks])
    assert np.allclose(r["O"][0], w @ v[toks])
    assert r["lse"][0] == pytest.approx(logsumexp(a[toks]))


def test_threshold_order_is_descending():
    """Visiting tile 0 first would set a low running max and keep tile 2; the
    descending walk (newest first) skips it."""
    q, k, v, a = _hand_example()
    r = orc.threshold_walk(q, k, v, np.array([7]), 2, 1e-3, 1.0, causal=False)
    assert list(r["decision"].keys()) == [3, 2, 1, 0]
    assert r["decision"][2] is False


def test_threshold_lambda_zero_is_dense_causal():
    rng = np.random.default_rng(13)
    L, D, T = 256, 16, 32
    q = rng.standard_normal((1, 2, L, D)) * 2
    k = rng.standard_normal((1, 1, L, D)) * 2
    v = rng.standard_normal((1, 1, L, D))
    p = dict(tile=T, causal=1, lam=0.0, scale=0.25)
    res = orc.threshold_attention(p, q, k, v, [(0, h, t) for h in range(2) for t in range(L // T)])
    for h in range(2):
        o2, l2 = _dense(q[0, h], k[0, 0], v[0, 0], 0.25, np.arange(L))
        for t in range(L // T):
            r = res[(0, h, t)]
            assert r["kept"] == list(range(t + 1))
            assert np.allclose(r["O"], o2[t * T:(t + 1) * T], atol=1e-12)
            assert np.allclose(r["lse"], l2[t * T:(t + 1) * T])


def test_threshold_skipped_mass_bound():
    """|O_lambda - O_dense| <= 2 max|v| M_skip / (M_kept + M_skip) per row."""
    w = synth.threshold_prefill(L=1024, Hq=1, Hkv=1, D=32, tile=32, seg_tiles=3, n_needles=1, logit_gap=6.0)
    q, k, v = w.f64("q")[0, 0], w.f64("k")[0, 0], w.f64("v")[0, 0]
    L, T, scale = 1024, 32, w.params["scale"]
    o_dense, _ = _dense(q, k, v, scale, np.arange(L))
    n_skipped, worst = 0, 0.0
    for t in range(L // T):
        rows = np.arange(t * T, (t + 1) * T)
        r = orc.threshold_walk(q[rows], k, v, rows, T, 0.02, scale)
        n_skipped += (t + 1) - len(r["kept"])
        bound = 2 * np.abs(v).max() * r["mass_skipped"] / (r["mass_kept"] + r["mass_skipped"])
        err = np.abs(r["O"] - o_dense[rows]).max(axis=1)
        assert np.all(err <= bound + 1e-12)
        worst = max(worst, float(err.max()))
    assert n_skipped > 0 and worst > 0


def test_threshold_decode_is_the_walk_per_head():
    """Decode runs the prefill walk on each head's single row; the hand example
    gives the same kept tiles through either entry."""
    q, k, v, a = _hand_example()
    for lam, kept in ((1e-3, [0, 1, 3]), (0.1, [3]), (0.04, [1, 3])):
        O, lse, keep, _ = orc.threshold_decode(q[None, :, None, :][:, 0:1], k[None, None], v[None, None], lam,
                                               1.0, 2)
        assert np.flatnonzero(keep[0, 0]).tolist() == kept
        toks = np.concatenate([[2 * j, 2 * j + 1] for j in kept])
        assert np.allclose(O[0, 0, 0], softmax(a[toks]) @ v[toks])
        assert lse[0, 0, 0] == pytest.approx(logsumexp(a[toks]))


def test_threshold_decisions_follow_the_prefix_max():
    """A skipped tile never raises the running max (it trails it by at least
    ln(1/lambda) >= 0), so the walk's max before tile j is the max over all
    newer tiles, kept or not: tile j is kept iff tm_j - max(tm_i, i > j) >=
    ln(lambda).  Checked by brute force against the sequential walk."""
    rng = np.random.default_rng(23)
    L, D, T = 64 * 40, 16, 64
    for trial in range(6):
        q = rng.standard_normal((1, 3, 1, D)) * (1 + trial)
        k = rng.standard_normal((1, 1, L, D))
        v = rng.standard_normal((1, 1, L, D))
        lam = (0.02, 0.2, 0.5, 0.8, 1.0, 1e-4)[trial]
        _, _, keep, _ = orc.threshold_decode(q, k, v, lam, 0.4, T)
        for h in range(3):
            s = 0.4 * (k[0, 0] @ q[0, h, 0])
            tm = s.reshape(-1, T).max(axis=1)
            newer = np.array([tm[j + 1:].max() if j + 1 < len(tm) else -np.inf for j in range(len(tm))])
            want = (newer == -np.inf) | (tm - newer >= math.log(lam))
            assert np.array_equal(keep[0, h], want), (trial, h)


def test_threshold_decode_lambda_zero_is_dense():
    rng = np.random.default_rng(21)
    L, D = 300, 16
    q = rng.standard_normal((2, 4, 1, D))
    k = rng.standard_normal((2, 2, L, D))
    v = rng.standard_normal((2, 2, L, D))
    O, lse, keep, _ = orc.threshold_decode(q, k, v, 0.0, 0.3, 32)
    assert keep.all()
    for b in range(2):
        for h in range(4):
            o2, l2 = _dense(q[b, h], k[b, h // 2], v[b, h // 2], 0.3)
            assert np.allclose(O[b, h], o2, atol=1e-12) and np.allclose(lse[b, h], l2)


def test_threshold_workload_skip_fraction_on_sample():
    """The planted local window gives about 70% skippable tiles; check the walk
    on a few query tiles of a reduced-width workload against the segment model."""
    w = synth.threshold_prefill(L=8192, Hq=2, Hkv=1, seg_tiles=7, n_needles=1)
    p = w.params
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    seg = w.extra["seg_tiles"]
    needle = int(w.extra["needles"][0, 0])
    for qt in (5, 20, 37, 50, 63):
        r = orc.threshold_attention(p, q, k, v, [(0, 0, qt)])[(0, 0, qt)]
        m = qt // seg
        window = set(range(max(0, (m - 1) * seg), qt + 1))
        if needle <= qt:
            window.add(needle)
        assert set(r["kept"]) == window


def test_threshold_rule_matches_the_blasst_golden():
    """The stored skip rule (BLASST technical summary sec. 2, with the prefill workload's
    "running max - ln(1e3)"): lambda = 1e-3, ln(lambda) as stored; a tile whose max trails the
    running max by just less than ln(1/lambda) is kept, by just more is skipped."""
    g = _golden("blasst_rule.txt")
    assert g["lambda"] == 1e-3 and g["ln_lambda"] == pytest.approx(math.log(g["lambda"]), abs=1e-15)
    assert synth.threshold_prefill(L=256, Hq=1, Hkv=1, D=16, tile=32, seg_tiles=2, n_needles=1).params["lam"] \
        == g["lambda"]
    v = np.random.default_rng(3).standard_normal((4, 4))
    for delta, kept in ((1e-6, [0, 1]), (-1e-6, [1])):
        # tile 1 (visited first) has max 0; tile 0's max trails it by |ln lambda| - delta
        a = np.array([g["ln_lambda"] + delta, g["ln_lambda"] - 5.0, 0.0, -1.0])
        q = np.zeros((1, 4)); q[0, 0] = 1.0
        k = np.zeros((4, 4)); k[:, 0] = a
        r = orc.threshold_walk(q, k, v, np.array([3]), 2, g["lambda"], 1.0, causal=False)
        assert r["kept"] == kept, (delta, r["kept"])
        assert r["margin"][0] == pytest.approx(delta, abs=1e-12)


@pytest.mark.parametrize("L", [64 * 5 + 19, 64 * 5, 64 * 4 + 1])
def test_decode_step_refreshes_only_the_newest_block(L):
    """decode_step pools exactly block (L - 1) // b from K (mean and both band energies), writes no
    other summary, and then equals selection + attention on the complete summaries.  L is ragged,
    an exact multiple of b, and one token into a new block."""
    rng = np.random.default_rng(L)
    B, Hq, Hkv, D, b = 1, 4, 2, 16, 64
    q = rng.standard_normal((B, Hq, 1, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    p = dict(kv_block=b, q_block=1, q_pos0=L - 1, causal=0, topk=2, topk_num=0, topk_den=1, n_first=1,
             n_last=1, dual_band=0, layout=ROPE_HALF, scale=1.0 / math.sqrt(D))
    NB = -(-L // b)
    j = (L - 1) // b
    t0 = j * b
    # the newest block's summary by its definition, written out here: mean and per-band mean energy
    fast = np.zeros(D, dtype=bool)
    fast[:D // 4] = True
    fast[D // 2:D // 2 + D // 4] = True
    seg = k[:, :, t0:L, :]
    mean_j = seg.sum(axis=2) / (L - t0)
    en_j = np.stack([(seg[..., fast] ** 2).sum(axis=(2, 3)), (seg[..., ~fast] ** 2).sum(axis=(2, 3))], -1) / (L - t0)
    # stale newest block; sentinel values elsewhere must come back untouched
    km = rng.standard_normal((B, Hkv, NB, D)) + 100.0
    ke = rng.standard_normal((B, Hkv, NB, 2)) + 100.0
    km_in, ke_in = km.copy(), ke.copy()
    orc.decode_step(p, q, k, v, km, ke)
    others = np.arange(NB) != j
    assert np.array_equal(km[:, :, others], km_in[:, :, others])
    assert np.array_equal(ke[:, :, others], ke_in[:, :, others])
    assert np.allclose(km[:, :, j], mean_j, atol=1e-12) and np.allclose(ke[:, :, j], en_j, atol=1e-12)
    # with correct older summaries the step equals the separate pieces on the full summaries
    km_full, ke_full = orc.block_summaries(k, b, ROPE_HALF)
    km2, ke2 = km_full.copy(), ke_full.copy()
    km2[:, :, j] = 0.0
    ke2[:, :, j] = 0.0
    O, LSE, lists = orc.decode_step(p, q, k, v, km2, ke2)
    assert np.allclose(km2, km_full, atol=1e-12) and np.allclose(ke2, ke_full, atol=1e-12)
    sel = orc.select_blocks(p, km_full, q=q)
    O2, L2 = orc.sparse_attention(p, q, k, v, sel["lists"])
    for g in range(Hkv):
        assert np.array_equal(lists[0][g][0], sel["lists"][0][g][0])
        assert len(lists[0][g][0]) == min(NB, 4) and {0, NB - 1} <= set(lists[0][g][0].tolist())
    assert np.allclose(O, O2, atol=1e-12) and np.allclose(LSE, L2, atol=1e-12)
    # and with every block listed it is dense attention over all L keys
    p_all = dict(p, topk=NB)
    O3, L3, _ = orc.decode_step(p_all, q, k, v, km_full.copy(), ke_full.copy())
    for h in range(Hq):
        o_d, l_d = _dense(q[0, h], k[0, h // 2], v[0, h // 2], p["scale"])
        assert np.allclose(O3[0, h], o_d, atol=1e-12) and np.allclose(L3[0, h], l_d)


# --------------------------------------------------------------- generators ---
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(15).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]   # exact ties and a subnormal
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((5, 16))
    pos = np.array([0, 1, 17, 1000, 65535])
    th = 10000.0 ** (-2.0 * np.arange(8) / 16)
    for layout in (ROPE_HALF, ROPE_INTERLEAVED):
        a, b = _fc_pairs(16, layout)
        z = (x[:, a] + 1j * x[:, b]) * np.exp(1j * pos[:, None] * th[None, :])
        y = synth.rope(x, pos, layout)
        assert np.allclose(y[:, a], z.real) and np.allclose(y[:, b], z.imag)


def test_generators_are_deterministic():
    a = synth.gqa_decode(L=1024, Hq=4, Hkv=1)
    b = synth.gqa_decode(L=1024, Hq=4, Hkv=1)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)


def test_decode_batch_shifts_give_distinct_whole_block_rolls():
    """The batched decode inputs: sequence 0 unshifted, every shift a distinct
    whole number of blocks, and shift_sequence is a circular roll along L (so
    block j of the base cache is block (j + s / block) mod NB of sequence b)."""
    L, block = 4096, 64
    NB = L // block
    sh = synth.decode_batch_shifts(32, L, block)
    assert sh[0] == 0 and len(set(sh)) == 32
    assert all(s % block == 0 and 0 <= s < L for s in sh)
    assert sh == synth.decode_batch_shifts(32, L, block)          # seeded
    x = np.arange(2 * L * 3, dtype=np.int64).reshape(2, L, 3)
    for s in sh[:4]:
        y = synth.shift_sequence(x, s)
        for j in (0, 5, NB - 1):
            jb = (j + s // block) % NB
            assert np.array_equal(y[:, jb * block:(jb + 1) * block], x[:, j * block:(j + 1) * block])
    with pytest.raises(ValueError):
        synth.decode_batch_shifts(4, L + 1, block)
