"""GPU vs fp64 oracle parity for every step of the hot path (needs an MI355X).

Each case generates seeded synthetic inputs, runs the HIP library through its
C ABI (via the thin binding) and checks the results against the oracle on the
same stored values: block summaries and energies, band temperatures, per-row
picks and per-block lists (tie band 1e-6), attention outputs and LSE, active
rows, and threshold keep/skip decisions.  Small cases span several tiles and
a ragged tail; the full-size cases use the shapes and launch configuration
the benchmark times, checked on sampled rows.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle as orc
import synth
from parity import (THRESH_EPS, ambiguous, check_list, check_outputs, check_row_picks, check_threshold_walk,
                    from_dev, record_threshold, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import dlm_bsa_block_amd as m
    m.lib()          # raises when libbsa.so is missing: never silently skipped on a GPU
    return m


def _sync():
    torch.cuda.synchronize()


def _f32_out(like):
    return torch.zeros(like.shape, dtype=torch.float32, device=like.device)


def _check_rounding(o_bf16, o_f32, rows=None):
    """The bf16 output is the f32 output rounded to nearest even, bit for bit
    (the same kernel with the other store).  The f32 output is what the oracle
    is compared with: the fp32 result before its final rounding, so that the
    output tolerance measures the computation and not the bf16 storage of
    values up to |O| ~ 4 (half an ulp there is 2^-7)."""
    a, b = o_bf16, o_f32.to(torch.bfloat16)
    if rows is not None:
        a, b = a[:, :, rows], b[:, :, rows]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "bf16 output is not the rounded f32 output"


# --------------------------------------------------------------- summaries ---
@pytest.mark.parametrize("dtype,D,L,block,layout", [
    ("bf16", 128, 1000, 64, 0), ("bf16", 128, 4000, 128, 1), ("f32", 64, 1024, 64, 0),
    ("bf16", 64, 777, 16, 1), ("f32", 128, 300, 256, 0), ("bf16", 128, 96, 32, 0)])
def test_summaries(bsa, dtype, D, L, block, layout):
    rng = np.random.default_rng(L + D)
    x64 = rng.standard_normal((2, 3, L, D)) * 1.5
    xs = synth.f32_to_bf16_bits(x64.astype(np.float32)) if dtype == "bf16" else x64.astype(np.float32)
    xr = synth.storage_to_f64(xs, dtype)
    xd = to_dev(xs, dtype)
    mean, energy = bsa.bsa_build_block_summaries(xd, block, layout)
    _sync()
    m_ref, e_ref = orc.block_summaries(xr, block, layout)
    assert np.allclose(from_dev(mean), m_ref, rtol=1e-5, atol=2e-6)
    assert np.allclose(from_dev(energy), e_ref, rtol=1e-5, atol=1e-5)
    # partial rebuild: only the newest block is written
    NB = m_ref.shape[2]
    mean2 = torch.full_like(mean, float("nan"))
    bsa.bsa_build_block_summaries(xd, block, layout, first_block=NB - 1, num_blocks=1, mean=mean2, energy=energy)
    _sync()
    m2 = from_dev(mean2)
    assert np.isnan(m2[:, :, :NB - 1]).all()
    assert np.allclose(m2[:, :, NB - 1], m_ref[:, :, NB - 1], rtol=1e-5, atol=2e-6)


def test_summaries_strided_view(bsa):
    """A [B, H, L, D] view with a padded row stride (e.g. a slice of a larger cache)."""
    rng = np.random.default_rng(5)
    big = synth.f32_to_bf16_bits(rng.standard_normal((1, 2, 512, 192)).astype(np.float32))
    xd = to_dev(big, "bf16")[:, :, :, 32:160]
    mean, _ = bsa.bsa_build_block_summaries(xd, 64, 0)
    _sync()
    m_ref, _ = orc.block_summaries(synth.storage_to_f64(big, "bf16")[:, :, :, 32:160], 64, 0)
    assert np.allclose(from_dev(mean), m_ref, rtol=1e-5, atol=2e-6)


# -------------------------------------------------------------- pipelines ---
def _dev_workload(w):
    return to_dev(w.q, w.dtype), to_dev(w.k, w.dtype), to_dev(w.v, w.dtype)


def _select_raw(bsa, w, qd, kmean, row_mask=None):
    p = w.params
    D = w.q.shape[3]
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=p["q_block"], q_pos0=p["q_pos0"], causal=p["causal"],
                           topk=p["topk"], topk_num=p["topk_num"], topk_den=p["topk_den"], n_first=p["n_first"],
                           n_last=p["n_last"], layout=p["layout"], scale=p["scale"], D=D)
    idx, cnt, rp, _ = bsa.bsa_select_blocks(qd, kmean, sp, row_mask=row_mask, want_row_picks=True)
    return idx, cnt, rp, sp.cap


def _check_selection(sel, idx, cnt, rp, rows_of_block, where):
    """Per-row picks with the tie band, then every list; returns the tie-band sizes."""
    idx, cnt, rp = idx.cpu().numpy(), cnt.cpu().numpy(), rp.cpu().numpy()
    bands = {}
    for (b, g, r), row in sel["rows"].items():
        check_row_picks(rp[b, g, r], row, f"{where} row b{b} g{g} r{r}")
    B, Hkv, NQB = cnt.shape
    n_tie = 0
    for b in range(B):
        for g in range(Hkv):
            for qb in range(NQB):
                band = set()
                for r in rows_of_block(qb):
                    if (b, g, r) in sel["rows"]:
                        band |= ambiguous(sel["rows"][(b, g, r)])
                n_tie += len(band)
                check_list(idx[b, g, qb], int(cnt[b, g, qb]), sel["lists"][b][g][qb], band, f"{where} list g{g} qb{qb}")
                bands[(b, g, qb)] = band
    return idx, cnt, n_tie


def _reference_lists(sel, idx, cnt):
    """The oracle's lists, except where the GPU's list differs inside the tie band
    (already checked): there either answer is correct and the GPU's is used."""
    B, Hkv, NQB = cnt.shape
    out = [[[None] * NQB for _ in range(Hkv)] for _ in range(B)]
    for b in range(B):
        for g in range(Hkv):
            for qb in range(NQB):
                gl = idx[b, g, qb, :cnt[b, g, qb]].astype(np.int64)
                ol = sel["lists"][b][g][qb]
                out[b][g][qb] = ol if np.array_equal(gl, ol) else gl
    return out


def _decode_case(bsa, w):
    p = w.params
    qd, kd, vd = _dev_workload(w)
    kmean, kenergy = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=cap, q_pos0=p["q_pos0"], causal=p["causal"],
                         scale=p["scale"])
    o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap)
    if qd.dtype == torch.bfloat16:
        o32, lse32 = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, o=_f32_out(qd))
        _sync()
        _check_rounding(o, o32)
        assert torch.equal(lse, lse32)
        o = o32
    _sync()
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    km_ref, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    assert np.allclose(from_dev(kmean), km_ref, rtol=1e-5, atol=2e-6)
    sel = orc.select_blocks(p, km_ref, q=q)
    idx_np, cnt_np, n_tie = _check_selection(sel, idx, cnt, rp, lambda qb: [qb], w.name)
    O_ref, L_ref = orc.sparse_attention(p, q, k, v, _reference_lists(sel, idx_np, cnt_np))
    stats = check_outputs(from_dev(o), O_ref, from_dev(lse), L_ref, w.name)
    return stats, idx_np, cnt_np, n_tie


def test_tiny_decode_exact_config(bsa):
    w = synth.tiny_decode()
    stats, idx, cnt, n_tie = _decode_case(bsa, w)
    assert cnt[0, 0, 0] == 4 and {0, 15} <= set(idx[0, 0, 0, :4].tolist())


@pytest.mark.parametrize("L", [8192, 8000, 1000])
def test_gqa_decode_small(bsa, L):
    w = synth.gqa_decode(L=L, n_needles=4)
    stats, idx, cnt, _ = _decode_case(bsa, w)
    NB = -(-L // 64)
    for g in range(8):
        lst = set(idx[0, g, 0, :cnt[0, g, 0]].tolist())
        assert len(lst) == 16 and {0, NB - 2, NB - 1} <= lst
        assert set(w.extra["needles"][g].tolist()) <= lst


def test_gqa_decode_full_size(bsa):
    """64K decode, 32 query / 8 KV heads: the benchmark's workload and launch."""
    w = synth.gqa_decode()
    stats, idx, cnt, _ = _decode_case(bsa, w)
    assert (cnt == 16).all()


def test_decode_select_everything_is_dense(bsa):
    """k' >= |C \\ F|: the list is every block, output equals dense attention."""
    w = synth.gqa_decode(L=2000, Hq=8, Hkv=2, n_needles=2)
    w.params.update(topk=1000)
    stats, idx, cnt, _ = _decode_case(bsa, w)
    assert (cnt == 32).all()


def _refresh_case(bsa, w):
    """Selection with the newest block's summary pooled inside it: the stored
    summary of that block is stale (zeros) before the call."""
    p = w.params
    qd, kd, vd = _dev_workload(w)
    NB = -(-kd.shape[2] // p["kv_block"])
    kmean, kenergy = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    kmean[:, :, NB - 1] = 0.0
    kenergy[:, :, NB - 1] = 0.0
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=1, q_pos0=p["q_pos0"], causal=p["causal"], topk=p["topk"],
                           n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"], scale=p["scale"])
    idx, cnt, rp = bsa.bsa_select_blocks_refresh(kd, NB - 1, qd, kmean, sp, k_energy=kenergy, want_row_picks=True)
    _sync()
    q, k = w.f64("q"), w.f64("k")
    km_ref, ke_ref = orc.block_summaries(k, p["kv_block"], p["layout"])
    assert np.allclose(from_dev(kmean), km_ref, rtol=1e-5, atol=2e-6)
    assert np.allclose(from_dev(kenergy), ke_ref, rtol=1e-5, atol=2e-6)
    sel = orc.select_blocks(p, km_ref, q=q)
    _check_selection(sel, idx, cnt, rp, lambda qb: [qb], w.name + " refresh")


@pytest.mark.parametrize("L", [4096 + 37, 8192])
def test_select_refresh_small(bsa, L):
    _refresh_case(bsa, synth.gqa_decode(L=L, n_needles=3))


def test_select_refresh_full_size(bsa):
    _refresh_case(bsa, synth.gqa_decode())


def _window_case(bsa, w, window, with_gates=True):
    """Selected blocks plus a sliding window of ``window`` keys in one pass,
    against the oracle's two branches on the same lists (checked first)."""
    p = w.params
    qd, kd, vd = _dev_workload(w)
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=cap, q_pos0=p["q_pos0"], causal=p["causal"],
                         scale=p["scale"])
    B, Hq, Lq, _ = qd.shape
    gates = None
    if with_gates:
        rng = np.random.default_rng(window)
        gates = torch.from_numpy(rng.uniform(0.1, 1.2, (B, Hq, Lq, 2)).astype(np.float32)).cuda()
    o32, lse = bsa.bsa_window_decode_fwd(qd, kd, vd, idx, cnt, ap, window, gates=gates, o=_f32_out(qd))
    if qd.dtype == torch.bfloat16:
        o16, lse16 = bsa.bsa_window_decode_fwd(qd, kd, vd, idx, cnt, ap, window, gates=gates, o=torch.empty_like(qd))
        _sync()
        _check_rounding(o16, o32)
        assert torch.equal(lse, lse16)
    _sync()
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    km_ref, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    sel = orc.select_blocks(p, km_ref, q=q)
    idx_np, cnt_np, _ = _check_selection(sel, idx, cnt, rp, lambda qb: [qb], w.name)
    g_np = None if gates is None else gates.cpu().numpy().astype(np.float64)
    O_ref, L_ref = orc.window_decode(p, q, k, v, _reference_lists(sel, idx_np, cnt_np), window, g_np)
    return check_outputs(from_dev(o32), O_ref, lse.cpu().numpy(), L_ref, f"{w.name} window {window}")


@pytest.mark.parametrize("L,window,gates", [(4096 + 37, 512, True), (4096 + 37, 300, False), (700, 5000, True),
                                            (2048, 64, True)])
def test_window_decode_small(bsa, L, window, gates):
    """Windows aligned and not to the blocks, longer than the prefix, one block long."""
    w = synth.gqa_decode(L=L, n_needles=2)
    _window_case(bsa, w, window, gates)


def test_window_decode_tiny_f32(bsa):
    """fp32 inputs, head dim 64, one head: the window branch through the fp32 decode path."""
    _window_case(bsa, synth.tiny_decode(), 100, True)


def test_token_attention_f32_lists(bsa):
    """Per-head token attention with fp32 inputs, head dim 64, group size 2, unsorted seeded lists of
    different lengths (one empty) -- the lists need not come from the token selection."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, L, D, cap = 2, 4, 2, 700, 64, 90
    q = rng.standard_normal((B, Hq, 1, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    idx = np.zeros((B, Hq, 1, cap), dtype=np.int32)
    cnt = np.zeros((B, Hq, 1), dtype=np.int32)
    lists = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            n = 0 if (b, h) == (1, 2) else int(rng.integers(1, cap + 1))
            t = rng.choice(L, n, replace=False)
            idx[b, h, 0, :n] = t
            cnt[b, h, 0] = n
            lists[b][h] = t.astype(np.int64)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o, lse = bsa.bsa_token_attention_fwd(qd, kd, vd, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                                         scale=0.125)
    _sync()
    O_ref, L_ref = orc.token_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), lists, 0.125)
    check_outputs(o.cpu().numpy(), O_ref, lse.cpu().numpy(), L_ref, "token attention f32")
    assert torch.all(o[1, 2] == 0) and lse[1, 2, 0].item() == float("-inf")


def test_window_decode_full_size(bsa):
    """64K decode with the page's window of 512 keys."""
    _window_case(bsa, synth.gqa_decode(), 512)


def _fp32_dot_bound(n_terms: int) -> float:
    """gamma_n = n u / (1 - n u), u = 2^-24: |fl(sum) - sum| <= gamma_n * sum |terms|
    for a sum of n exact products accumulated in fp32 in any order."""
    nu = n_terms * 2.0 ** -24
    return nu / (1.0 - nu)


def _fc_mask(Hq, n_fc, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((Hq, 64), dtype=np.uint8)
    for h in range(Hq):
        m[h, rng.choice(64, n_fc, replace=False)] = 1
    return m


def _token_case(bsa, w, budget, n_fc, layout, seed=0):
    """Token scores on a subset of frequency chunks, top-N per head, then each
    head's attention over its own tokens, against the oracle."""
    p = w.params
    qd, kd, vd = _dev_workload(w)
    B, Hq = qd.shape[:2]
    L = kd.shape[2]
    mask = _fc_mask(Hq, n_fc, seed)
    idx, cnt = bsa.bsa_token_select(qd, kd, torch.from_numpy(mask).cuda(), budget, layout=layout)
    o32, lse = bsa.bsa_token_attention_fwd(qd, kd, vd, idx, cnt, scale=p["scale"], o=_f32_out(qd))
    o16, lse16 = bsa.bsa_token_attention_fwd(qd, kd, vd, idx, cnt, scale=p["scale"], o=torch.empty_like(qd))
    _sync()
    _check_rounding(o16, o32)
    assert torch.equal(lse, lse16)
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    S = orc.token_scores(q, k, mask, layout)
    # per-token rounding bound of the GPU's fp32 score: the sum of |products| over the kept dims,
    # times gamma_n, plus one rounding of the scaled result
    A = orc.token_scores(np.abs(q), np.abs(k), mask, layout)
    gam = _fp32_dot_bound(2 * n_fc)
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    n = min(budget, L)
    lists = [[None] * Hq for _ in range(B)]
    n_amb = 0
    for b in range(B):
        for h in range(Hq):
            assert cnt_np[b, h] == n
            got = idx_np[b, h, :n].astype(np.int64)
            assert np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < L, f"head {h}: list not ascending"
            ref, kth = orc.top_tokens(S[b, h], budget)
            # tokens whose exact score could fall on either side of the N-th one's after fp32 rounding
            ki = ref[np.argmin(S[b, h][ref])]
            band = gam * (A[b, h] + A[b, h][ki]) + 2.0 ** -23 * np.maximum(np.abs(S[b, h]), abs(kth))
            amb = set(np.nonzero(np.abs(S[b, h] - kth) <= band)[0].tolist())
            n_amb += len(amb)
            assert set(got.tolist()) - amb == set(ref.tolist()) - amb, f"head {h}: token sets differ"
            lists[b][h] = got
    O_ref, L_ref = orc.token_attention(q, k, v, lists, p["scale"])
    check_outputs(from_dev(o32), O_ref, lse.cpu().numpy(), L_ref, f"{w.name} tokens {budget}")
    return idx_np, n_amb


@pytest.mark.parametrize("L,budget,n_fc,layout", [(4096, 256, 8, 0), (3000 + 3, 100, 4, 1), (500, 1000, 64, 0),
                                                  (8192, 1, 16, 0)])
def test_token_select_small(bsa, L, budget, n_fc, layout):
    """Budgets below and above L (all tokens), one token, all chunks, both layouts, a ragged L."""
    w = synth.gqa_decode(L=L, n_needles=2)
    _token_case(bsa, w, budget, n_fc, layout, seed=L)


def test_token_select_group_size_8(bsa):
    w = synth.gqa_decode(L=2048, Hq=16, Hkv=2, n_needles=2)
    _token_case(bsa, w, 128, 8, 0, seed=3)


def test_token_select_full_size(bsa):
    """64K decode, 8 of 64 chunks per head, 256 tokens per head (the page's LongBench budget)."""
    idx, _ = _token_case(bsa, synth.gqa_decode(), 256, 8, 0, seed=64)
    assert idx.shape == (1, 32, 256)


def _dlm_case(bsa, w, union_active: bool, full_check_rows=None):
    p = w.params
    qd, kd, vd = _dev_workload(w)
    qprev = to_dev(w.extra["q_prev"], "bf16")
    mask, mse = bsa.bsa_active_rows(qd, qprev, p["theta_act"])
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean, row_mask=mask if union_active else None)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=p["q_block"], cap=cap, q_pos0=p["q_pos0"],
                         causal=p["causal"], scale=p["scale"])
    # cached outputs of the previous step: any values; stable rows must keep them bit for bit
    cache_o = torch.randn(qd.shape, device="cuda").to(torch.bfloat16)
    cache_l = torch.randn(qd.shape[:3], device="cuda")
    o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, row_mask=mask, o=cache_o.clone(),
                                          lse=cache_l.clone())
    o32, lse32 = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, row_mask=mask, o=cache_o.float(),
                                              lse=cache_l.clone())
    _sync()
    act_rows = torch.nonzero(mask[0]).flatten()
    _check_rounding(o, o32, act_rows)
    assert torch.equal(lse, lse32)
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    m_ref, mse_ref = orc.active_rows(q, w.f64("q_prev"), p["theta_act"])
    assert np.array_equal(mask.cpu().numpy().astype(bool), m_ref)
    assert np.allclose(mse.cpu().numpy(), mse_ref, rtol=1e-5)
    km_ref, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    sel = orc.select_blocks(p, km_ref, q=q, row_mask=m_ref if union_active else None)
    R = p["q_block"]
    idx_np, cnt_np, _ = _check_selection(sel, idx, cnt, rp, lambda qb: range(qb * R, (qb + 1) * R), w.name)
    O_ref, L_ref = orc.sparse_attention(p, q, k, v, _reference_lists(sel, idx_np, cnt_np), row_mask=m_ref)
    act = np.nonzero(m_ref[0])[0]
    o_np, l_np = from_dev(o32), lse.cpu().numpy()
    stats = check_outputs(o_np[:, :, act], O_ref[:, :, act], l_np[:, :, act], L_ref[:, :, act], w.name)
    stable = np.nonzero(~m_ref[0])[0]
    assert torch.equal(o[:, :, stable], cache_o[:, :, stable])
    assert torch.equal(lse[:, :, stable], cache_l[:, :, stable])
    return stats, cnt_np


@pytest.mark.parametrize("union_active", [False, True])
def test_dlm_denoise_small(bsa, union_active):
    w = synth.dlm_denoise(L=4096 + 100, n_needles=4)
    _dlm_case(bsa, w, union_active)


def test_dlm_denoise_full_size(bsa):
    w = synth.dlm_denoise()
    _, cnt_all = _dlm_case(bsa, w, False)
    _, cnt_act = _dlm_case(bsa, w, True)
    assert (cnt_act <= cnt_all).all() and (cnt_act < cnt_all).any()


def test_dlm_no_active_rows_writes_nothing(bsa):
    w = synth.dlm_denoise(L=2048, n_needles=2)
    p = w.params
    qd, kd, vd = _dev_workload(w)
    kmean, _ = bsa.bsa_build_block_summaries(kd, 64, 0)
    mask = torch.zeros((1, 32), dtype=torch.uint8, device="cuda")
    idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean, row_mask=mask)
    ap = bsa.attn_params(kv_block=64, q_block=32, cap=cap, q_pos0=p["q_pos0"])
    o0 = torch.randn(qd.shape, device="cuda").to(torch.bfloat16)
    o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, row_mask=mask, o=o0.clone())
    _sync()
    assert (cnt == 0).all() and torch.equal(o, o0)
    assert (rp == -1).all()


# ------------------------------------------------- merge and full denoise ---
def test_merge_states(bsa):
    """bsa_merge_attention_states against the oracle's union-of-key-sets merge:
    mixed input dtypes, empty states (LSE -inf, O ignored), rows empty on both
    sides, a ragged row count, in place into one of the inputs."""
    rng = np.random.default_rng(21)
    shape = (2, 3, 37, 128)
    oa = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda().to(torch.bfloat16)
    ob = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * 3).cuda()
    la = rng.uniform(-5, 25, shape[:3]).astype(np.float32)
    lb = rng.uniform(-5, 25, shape[:3]).astype(np.float32)
    la[0, 0, :5] = -np.inf
    lb[1, 2, 3:9] = -np.inf
    la[1, 1, 10:12] = lb[1, 1, 10:12] = -np.inf
    lb[0, 1, 20] = la[0, 1, 20] + 40.0             # one side dominates
    oa[0, 0, :5] = float("nan")                      # O of an empty state is never read into the result
    ob[1, 2, 3:9] = float("nan")
    lad, lbd = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    o32, l32 = bsa.bsa_merge_attention_states(oa, lad, ob, lbd, o=torch.empty(shape, device="cuda"))
    o16, l16 = bsa.bsa_merge_attention_states(oa, lad, ob, lbd, o=torch.empty(shape, device="cuda",
                                                                               dtype=torch.bfloat16))
    ob_in, lb_in = ob.clone(), lbd.clone()
    bsa.bsa_merge_attention_states(oa, lad, ob_in, lb_in, o=ob_in, lse=lb_in)
    _sync()
    oa64 = oa.float().cpu().numpy().astype(np.float64)
    ob64 = ob.cpu().numpy().astype(np.float64)
    oa64[0, 0, :5] = 0.0                             # the oracle is given finite values where the GPU gets NaN
    ob64[1, 2, 3:9] = 0.0
    O_ref, L_ref = orc.merge_states(oa64, la.astype(np.float64), ob64, lb.astype(np.float64))
    o_np, l_np = o32.cpu().numpy(), l32.cpu().numpy()
    assert np.array_equal(np.isinf(l_np), np.isinf(L_ref))
    fin = np.isfinite(L_ref)
    assert np.abs(l_np[fin] - L_ref[fin]).max() < 1e-5
    assert np.abs(o_np - O_ref).max() < 2e-5
    assert np.all(o_np[1, 1, 10:12] == 0)
    assert torch.equal(l16, l32)
    _check_rounding(o16, o32)
    assert torch.equal(ob_in, o32) and torch.equal(lb_in, l32), "in-place merge differs"


def _denoise_loop(bsa, w, check=True):
    """Run the denoising steps of ``w`` through the library: step 0 dense over
    the prefix for every row, later steps sparse for the active rows only
    (union over them), stable rows keeping their cached prefix state, and every
    row merged with its attention over the block's own keys.  With ``check``
    each step is compared with the oracle's step (lists first, with the tie
    band).  Returns the per-step active-row counts and list sizes."""
    p = w.params
    B, Hq, R, D = w.q.shape
    Hkv, L = w.k.shape[1], w.k.shape[2]
    NB = -(-L // p["kv_block"])
    kd, vd = to_dev(w.k, "bf16"), to_dev(w.v, "bf16")
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    cache_o = torch.zeros((B, Hq, R, D), device="cuda")
    cache_l = torch.zeros((B, Hq, R), device="cuda")
    idx_in = torch.zeros((B, Hkv, 1, 1), dtype=torch.int32, device="cuda")
    cnt_in = torch.ones((B, Hkv, 1), dtype=torch.int32, device="cuda")
    ap_in = bsa.attn_params(kv_block=64, q_block=R, cap=1, q_pos0=0, causal=0, scale=p["scale"])
    if check:
        k64, v64 = w.f64("k"), w.f64("v")
        km_ref, _ = orc.block_summaries(k64, p["kv_block"], p["layout"])
        rO, rL = np.zeros((B, Hq, R, D)), np.zeros((B, Hq, R))
    stats = []
    qprev = None
    for s, (qs, kbs, vbs) in enumerate(zip(w.extra["q_steps"], w.extra["kb_steps"], w.extra["vb_steps"])):
        where = f"{w.name} step {s}"
        qd, kbd, vbd = to_dev(qs, "bf16"), to_dev(kbs, "bf16"), to_dev(vbs, "bf16")
        if s == 0:
            mask = None
            cnt = torch.full((B, Hkv, 1), NB, dtype=torch.int32, device="cuda")
            idx = torch.arange(NB, dtype=torch.int32, device="cuda").view(1, 1, 1, NB).repeat(B, Hkv, 1, 1)
            cap = NB
        else:
            mask, _ = bsa.bsa_active_rows(qd, qprev, p["theta_act"])
            idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean, row_mask=mask)
        ap = bsa.attn_params(kv_block=p["kv_block"], q_block=R, cap=cap, q_pos0=p["q_pos0"], causal=0,
                             scale=p["scale"])
        bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, row_mask=mask, o=cache_o, lse=cache_l)
        # the fused block attention + merge, and the same from the general pieces (the block as a
        # one-block sparse attention, then the state merge)
        o32, l32 = bsa.bsa_block_attention_merge(qd, kbd, vbd, cache_o, cache_l, scale=p["scale"], o=_f32_out(qd))
        o16, l16 = bsa.bsa_block_attention_merge(qd, kbd, vbd, cache_o, cache_l, scale=p["scale"],
                                                 o=torch.empty_like(qd))
        o_in, l_in = bsa.bsa_sparse_attention_fwd(qd, kbd, vbd, idx_in, cnt_in, ap_in, o=_f32_out(qd))
        o32b, l32b = bsa.bsa_merge_attention_states(cache_o, cache_l, o_in, l_in, o=_f32_out(qd))
        o_ip, l_ip = cache_o.clone(), cache_l.clone()
        bsa.bsa_block_attention_merge(qd, kbd, vbd, o_ip, l_ip, scale=p["scale"], o=o_ip, lse=l_ip)
        _sync()
        assert torch.equal(o_ip, o32) and torch.equal(l_ip, l32), f"{w.name} step {s}: in-place merge differs"
        n_act = R if mask is None else int(mask.sum().item())
        stats.append(dict(active=n_act, list_blocks=cnt[0, :, 0].cpu().tolist()))
        if check:
            q64 = synth.storage_to_f64(qs, "bf16")
            kb64, vb64 = synth.storage_to_f64(kbs, "bf16"), synth.storage_to_f64(vbs, "bf16")
            if s == 0:
                m_ref, lists = None, [[[np.arange(NB)] for _ in range(Hkv)] for _ in range(B)]
            else:
                m_ref, _ = orc.active_rows(q64, synth.storage_to_f64(w.extra["q_steps"][s - 1], "bf16"),
                                           p["theta_act"])
                assert np.array_equal(mask.cpu().numpy().astype(bool), m_ref), where
                assert np.array_equal(np.nonzero(m_ref[0])[0], w.extra["changed"][s]), where
                sel = orc.select_blocks(p, km_ref, q=q64, row_mask=m_ref)
                idx_np, cnt_np, _ = _check_selection(sel, idx, cnt, rp, lambda qb: range(qb * R, (qb + 1) * R),
                                                     where)
                lists = _reference_lists(sel, idx_np, cnt_np)
            O_ref, L_ref, rO, rL = orc.denoise_step(p, q64, k64, v64, kb64, vb64, lists, m_ref, rO, rL)
            check_outputs(from_dev(o32), O_ref, l32.cpu().numpy(), L_ref, where)
            check_outputs(from_dev(o32b), O_ref, l32b.cpu().numpy(), L_ref, where + " (general pieces)")
            assert torch.equal(l16, l32)
            _check_rounding(o16, o32)
        qprev = qd
    return stats


def test_denoise_steps_small(bsa):
    """Four steps over a 2152-token prefix (34 blocks, the last ragged)."""
    w = synth.dlm_denoise_steps(L=2048 + 64 + 40, n_needles=2, n_steps=4)
    st = _denoise_loop(bsa, w)
    assert st[0]["active"] == 32 and all(x["active"] == 4 for x in st[1:])


@pytest.mark.parametrize("R,Hq,Hkv", [(20, 16, 4), (16, 16, 2)])
def test_denoise_steps_short_block(bsa, R, Hq, Hkv):
    """Blocks of fewer rows than the block attention's 32 key lanes; group sizes 4 and 8."""
    w = synth.dlm_denoise_steps(L=1024 + 7, R=R, Hq=Hq, Hkv=Hkv, n_needles=2, n_steps=3, per_step=3)
    st = _denoise_loop(bsa, w)
    assert all(x["active"] == 3 for x in st[1:])


def test_denoise_steps_full_size(bsa):
    """The benchmark's 32K prefix, first three steps (dense, then two sparse)."""
    w = synth.dlm_denoise_steps(n_steps=3)
    st = _denoise_loop(bsa, w)
    assert all(max(x["list_blocks"]) < 512 for x in st[1:])


def _prefill_case(bsa, w, sample_qb=None):
    p = w.params
    qd, kd, vd = _dev_workload(w)
    b = p["kv_block"]
    qmean, qen = bsa.bsa_build_block_summaries(qd, b, p["layout"])
    kmean, ken = bsa.bsa_build_block_summaries(kd, b, p["layout"])
    Lq = w.q.shape[2]
    sp = bsa.select_params(kv_block=b, q_block=p["q_block"], q_pos0=0, q_len=Lq, causal=1, pooled_q=1,
                           topk_num=p["topk_num"], topk_den=p["topk_den"], n_first=p["n_first"], n_last=p["n_last"],
                           dual_band=1, layout=p["layout"], scale=p["scale"])
    idx, cnt, rp, tau = bsa.bsa_select_blocks(qmean, kmean, sp, k_energy=ken, q_energy=qen, want_row_picks=True,
                                              want_tau=True)
    ap = bsa.attn_params(kv_block=b, q_block=p["q_block"], cap=sp.cap, q_pos0=0, causal=1, scale=p["scale"])
    o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap)
    o32, lse32 = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, o=_f32_out(qd))
    _sync()
    _check_rounding(o, o32)
    assert torch.equal(lse, lse32)
    o = o32
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    qm_ref, qe_ref = orc.block_summaries(q, b, p["layout"])
    km_ref, ke_ref = orc.block_summaries(k, b, p["layout"])
    assert np.allclose(from_dev(qmean), qm_ref, rtol=1e-5, atol=2e-6)
    assert np.allclose(from_dev(ken), ke_ref, rtol=1e-5, atol=1e-5)
    G = w.q.shape[1] // w.k.shape[1]
    tau_ref = orc.band_temperatures(km_ref, ke_ref, p["layout"], G, qm_ref, qe_ref)
    assert np.allclose(tau.cpu().numpy(), tau_ref, rtol=2e-5)
    sel = orc.select_blocks(p, km_ref, q_mean=qm_ref, tau=tau_ref, Lq=Lq)
    idx_np, cnt_np, n_tie = _check_selection(sel, idx, cnt, rp, lambda qb: [qb], w.name)
    NQB = cnt_np.shape[2]
    qbs = list(range(NQB)) if sample_qb is None else sample_qb
    O_ref, L_ref = orc.sparse_attention(p, q, k, v, _reference_lists(sel, idx_np, cnt_np), qblocks=qbs)
    rows = np.concatenate([np.arange(i * b, min((i + 1) * b, Lq)) for i in qbs])
    stats = check_outputs(from_dev(o)[:, :, rows], O_ref[:, :, rows], lse.cpu().numpy()[:, :, rows],
                          L_ref[:, :, rows], w.name)
    return stats, cnt_np


@pytest.mark.parametrize("L", [4096, 4000])
def test_sparse_prefill_small(bsa, L):
    w = synth.sparse_prefill(L=L, Hq=8, Hkv=2)
    stats, cnt = _prefill_case(bsa, w)
    NQB = cnt.shape[2]
    for i in range(NQB):
        assert cnt[0, 0, i] == min(i + 1, (2 if i else 1) + -(-(i + 1) // 10))


def test_sparse_prefill_group8(bsa):
    """Eight query heads per KV head: 16 (head, band) channels in the pick."""
    w = synth.sparse_prefill(L=4096, Hq=16, Hkv=2)
    _prefill_case(bsa, w)


def test_sparse_prefill_odd_group(bsa):
    """Odd group size (3 query heads per KV head) takes the one-head-per-workgroup
    path with 64-key tiles; ragged tail (2944 = 23 blocks of 128)."""
    w = synth.sparse_prefill(L=2944, Hq=3, Hkv=1)
    _prefill_case(bsa, w)


def test_sparse_prefill_full_size(bsa):
    """32K causal prefill, 32/8 heads: selection on every query block, outputs on 16 sampled blocks."""
    w = synth.sparse_prefill()
    rng = np.random.default_rng(4)
    sample = sorted(set([0, 255] + rng.choice(256, 14, replace=False).tolist()))
    stats, cnt = _prefill_case(bsa, w, sample_qb=sample)
    assert int(cnt[0].sum(axis=1)[0]) == 3915


@pytest.mark.parametrize("B,Hkv,G", [(2, 64, 2), (1, 32, 4)])
def test_prefill_handmade_lists(bsa, B, Hkv, G):
    """Causal gather attention on hand-made lists: several work items per
    workgroup of the streaming kernel (many KV groups, few CUs each), empty
    lists, blocks after the query block (wholly masked tiles), a ragged last
    query block (1000 = 7 * 128 + 104)."""
    L, D, blk = 1000, 128, 128
    NB = -(-L // blk)
    rng = np.random.default_rng(17 + G)
    Hq = Hkv * G
    qs, ks, vs = (synth.f32_to_bf16_bits(rng.standard_normal((B, h, L, D), dtype=np.float32))
                  for h in (Hq, Hkv, Hkv))
    lists = [[[None] * NB for _ in range(Hkv)] for _ in range(B)]
    idx = np.full((B, Hkv, NB, NB), -1, np.int32)
    cnt = np.zeros((B, Hkv, NB), np.int32)
    for b in range(B):
        for g in range(Hkv):
            for qb in range(NB):
                cand = np.arange(min(NB, qb + 2))
                n = 0 if rng.random() < 0.125 else int(rng.integers(1, len(cand) + 1))
                sel = np.sort(rng.choice(cand, n, replace=False)).astype(np.int64)
                lists[b][g][qb] = sel
                idx[b, g, qb, :n] = sel
                cnt[b, g, qb] = n
    assert (cnt == 0).any() and (cnt == np.minimum(NB, np.arange(NB) + 2)).any()
    ap = bsa.attn_params(kv_block=blk, q_block=blk, cap=NB, q_pos0=0, causal=1)
    args = (to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16"), torch.from_numpy(idx).cuda(),
            torch.from_numpy(cnt).cuda(), ap)
    o, lse = bsa.bsa_sparse_attention_fwd(*args)
    o32, lse32 = bsa.bsa_sparse_attention_fwd(*args, o=_f32_out(args[0]))
    _sync()
    _check_rounding(o, o32)
    assert torch.equal(lse, lse32)
    o = o32
    p = dict(kv_block=blk, q_block=blk, q_pos0=0, causal=1, scale=ap.scale)
    O_ref, L_ref = orc.sparse_attention(p, synth.storage_to_f64(qs, "bf16"), synth.storage_to_f64(ks, "bf16"),
                                        synth.storage_to_f64(vs, "bf16"), lists)
    check_outputs(from_dev(o), O_ref, lse.cpu().numpy(), L_ref, f"handmade B={B} Hkv={Hkv} G={G}")


# --------------------------------------------------------- threshold decode ---
def _threshold_decode_case(bsa, w, lam, kv_split, where):
    """GPU keep map replayed in the fp64 walk: each choice must agree with the
    fp64 margin outside THRESH_EPS; outputs are then compared with the replay."""
    qd, kd, vd = _dev_workload(w)
    scale = w.params["scale"]
    o, lse, kept, km = bsa.bsa_threshold_decode_fwd(qd, kd, vd, lam, scale=scale, kv_split=kv_split,
                                                    want_keep_map=True)
    o32, lse32, kept32, _ = bsa.bsa_threshold_decode_fwd(qd, kd, vd, lam, scale=scale, kv_split=kv_split,
                                                         o=_f32_out(qd))
    _sync()
    _check_rounding(o, o32)
    assert torch.equal(lse, lse32) and torch.equal(kept, kept32)
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    gkeep = km.cpu().numpy().astype(bool)
    assert np.array_equal(gkeep.sum(axis=2), kept.cpu().numpy()), f"{where}: kept counts disagree with the map"
    O_ref, L_ref, _, margin = orc.threshold_decode(q, k, v, lam, scale, 64, decisions=gkeep)
    differ = gkeep != (margin >= 0)
    bad = differ & (np.abs(margin) > THRESH_EPS)
    assert not bad.any(), f"{where}: {int(bad.sum())} keep/skip choices disagree with the fp64 walk"
    record_threshold(gkeep.size, int(differ.sum()), gkeep.shape[0] * gkeep.shape[1], 0,
                     float(np.abs(margin[differ]).max()) if differ.any() else 0.0)
    check_outputs(from_dev(o32), O_ref, lse.cpu().numpy(), L_ref, where)
    return float(1.0 - gkeep.mean())


@pytest.mark.parametrize("L,lam,kv_split", [(4096, 0.0, 1024), (4096, 0.3, 1024), (4096, 0.6, 256),
                                            (3000, 0.3, 512), (3000, 1.0, 2048), (3001, 0.3, 64)])
def test_threshold_decode_small(bsa, L, lam, kv_split):
    """Ragged slices and tiles (3000 = 46 tiles of 64 + 56; 3001), lambda from 0 (keep
    all) to 1 (keep only tiles that raise the running max); the decisions do
    not depend on the slicing, which only spreads the work."""
    w = synth.gqa_decode(L=L, n_needles=2)
    skipped = _threshold_decode_case(bsa, w, lam, kv_split, f"threshold decode L={L} lam={lam}")
    if lam == 0.0:
        assert skipped == 0.0
    else:
        assert skipped > 0.0


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (2, 2)])
def test_threshold_decode_group_sizes(bsa, Hq, Hkv):
    w = synth.gqa_decode(L=2048, Hq=Hq, Hkv=Hkv, n_needles=2)
    _threshold_decode_case(bsa, w, 0.4, 512, f"threshold decode G={Hq // Hkv}")


@pytest.mark.parametrize("which", ["calibrated", "aggressive"])
def test_threshold_decode_full_size(bsa, which):
    """64K decode, every head, at the benchmark's slices: the cache with the
    threshold-prefill structure at the calibrated lambda = a / L (the benchmark's
    configuration), and the flat GQA decode cache at lambda = 0.4, which skips
    most of its tiles (the skip path at full size)."""
    import bench
    if which == "calibrated":
        w = synth.threshold_decode(L=65536)
        lam = min(1.0, bench.THRESH_DECODE_A / w.k.shape[2])
    else:
        w, lam = synth.gqa_decode(), 0.4
    skipped = _threshold_decode_case(bsa, w, lam, bench.THRESH_DECODE_SPLIT, f"threshold decode 64K lam={lam:g}")
    if which == "aggressive":
        assert skipped > 0.3


# --------------------------------------------------------------- threshold ---
def _threshold_case(bsa, w, lam, pairs):
    """The GPU's keep map and outputs for the sampled (batch, head, query tile)
    triples, each checked against the fp64 walk (checks.check_threshold_walk:
    the walk is replayed on the GPU's choices when they differ inside the
    rounding band)."""
    p = w.params
    qd, kd, vd = _dev_workload(w)
    o, lse, kept, km = bsa.bsa_threshold_attention_fwd(qd, kd, vd, lam, scale=p["scale"], tile=p["tile"],
                                                       causal=p["causal"], want_keep_map=True)
    o32, lse32, kept32, _ = bsa.bsa_threshold_attention_fwd(qd, kd, vd, lam, scale=p["scale"], tile=p["tile"],
                                                            causal=p["causal"], o=_f32_out(qd))
    _sync()
    _check_rounding(o, o32)
    assert torch.equal(lse, lse32) and torch.equal(kept, kept32)
    o = o32
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    km_np, kept_np = km.cpu().numpy(), kept.cpu().numpy()
    o_np, l_np = from_dev(o), lse.cpu().numpy()
    G = w.q.shape[1] // w.k.shape[1]
    T = p["tile"]
    Lq = w.q.shape[2]
    tot = [0, 0, 0, 0.0]
    for (b, h, qt) in pairs:
        jmax = min(Lq - 1, (qt + 1) * T - 1) // T
        dec = {j: bool(km_np[b, h, qt, j]) for j in range(jmax + 1)}
        rows = np.arange(qt * T, min((qt + 1) * T, Lq))
        d, f, r, m = check_threshold_walk(q[b, h, rows], k[b, h // G], v[b, h // G], rows, T, lam, p["scale"],
                                          bool(p["causal"]), dec, kept_np[b, h, qt], o_np[b, h, rows],
                                          l_np[b, h, rows], f"thr h{h} qt{qt}")
        tot = [tot[0] + d, tot[1] + f, tot[2] + r, max(tot[3], m)]
    record_threshold(tot[0], tot[1], len(pairs), tot[2], tot[3])
    return kept_np, tot[2]


@pytest.mark.parametrize("L,lam", [(4096, 1e-3), (4000, 1e-3), (2048, 0.0), (4096, 0.3)])
def test_threshold_small(bsa, L, lam):
    w = synth.threshold_prefill(L=L, Hq=8, Hkv=2, seg_tiles=5, n_needles=2)
    NQT = -(-L // 128)
    pairs = [(0, h, qt) for h in (0, 3, 5) for qt in range(NQT)]
    kept, _ = _threshold_case(bsa, w, lam, pairs)
    if lam == 0.0:
        assert np.array_equal(kept[0, 0], np.arange(1, NQT + 1))


def test_threshold_odd_group(bsa):
    """Odd group size: one head per workgroup; ragged tail."""
    L = 1900
    w = synth.threshold_prefill(L=L, Hq=3, Hkv=1, seg_tiles=5, n_needles=2)
    NQT = -(-L // 128)
    _threshold_case(bsa, w, 1e-3, [(0, h, qt) for h in range(3) for qt in range(NQT)])


def test_threshold_full_size_sampled(bsa):
    """128K causal prefill with lambda = 1e-3, every one of the 32 heads: 16 query
    tiles per head (the last tile, which sees all 1024 KV tiles, and 15 drawn at
    random), walked in the fp64 oracle by one spawned CPU worker per KV group."""
    import multiprocessing as mp

    import threshold_walks
    w = synth.threshold_prefill()
    p = w.params
    T, lam = p["tile"], 1e-3
    Hq, Hkv = w.q.shape[1], w.k.shape[1]
    G, NQT = Hq // Hkv, -(-w.q.shape[2] // T)
    qd, kd, vd = _dev_workload(w)
    o, lse, kept, km = bsa.bsa_threshold_attention_fwd(qd, kd, vd, lam, scale=p["scale"], tile=T, causal=p["causal"],
                                                       o=_f32_out(qd), want_keep_map=True)
    _sync()
    kept_np = kept.cpu().numpy()
    sys.__stderr__.write("[threshold 128K] GPU pass done; gathering the sampled tiles\n")
    sys.__stderr__.flush()
    frac_skip = 1.0 - kept_np[0].sum() / (Hq * NQT * (NQT + 1) / 2)
    assert 0.66 < frac_skip < 0.74, frac_skip
    rng = np.random.default_rng(5)
    tasks = []
    for g in range(Hkv):
        items = []
        for h in range(g * G, (g + 1) * G):
            qts = [NQT - 1] + sorted(rng.choice(NQT - 1, 15, replace=False).tolist())
            for qt in qts:
                r0, r1 = qt * T, min((qt + 1) * T, w.q.shape[2])
                items.append(dict(h=h, qt=qt, q=np.ascontiguousarray(w.q[0, h, r0:r1]),
                                  dec={j: bool(x) for j, x in enumerate(km[0, h, qt, :qt + 1].cpu().numpy())},
                                  kept=int(kept_np[0, h, qt]), o=o[0, h, r0:r1].cpu().numpy(),
                                  lse=lse[0, h, r0:r1].cpu().numpy()))
        tasks.append(dict(k=np.ascontiguousarray(w.k[0, g]), v=np.ascontiguousarray(w.v[0, g]), tile=T, lam=lam,
                          scale=p["scale"], causal=bool(p["causal"]), items=items))
    del o, lse, km
    # one worker per KV group with two BLAS threads each: 16 threads, the CPU share of one GPU
    nproc = min(Hkv, 8)
    saved = {e: os.environ.get(e) for e in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for e in saved:
        os.environ[e] = "2"
    try:
        with mp.get_context("spawn").Pool(nproc) as pool:
            tot, walks = [0, 0, 0, 0.0], 0
            for (d, f, r, m), n in pool.imap_unordered(threshold_walks.check_group, tasks):
                tot = [tot[0] + d, tot[1] + f, tot[2] + r, max(tot[3], m)]
                walks += n
                sys.__stderr__.write(f"[threshold 128K] {walks} of {Hq * 16} walks checked\n")
                sys.__stderr__.flush()
    finally:
        for e, val in saved.items():
            if val is None:
                os.environ.pop(e, None)
            else:
                os.environ[e] = val
    assert walks == Hq * 16
    record_threshold(tot[0], tot[1], walks, tot[2], tot[3])


# ------------------------------------------------------------- determinism ---
def test_bitwise_repeatable(bsa):
    w = synth.sparse_prefill(L=2048, Hq=8, Hkv=2)
    outs = []
    for _ in range(2):
        qd, kd, vd = _dev_workload(w)
        p = w.params
        qmean, qen = bsa.bsa_build_block_summaries(qd, 128, p["layout"])
        kmean, ken = bsa.bsa_build_block_summaries(kd, 128, p["layout"])
        sp = bsa.select_params(kv_block=128, q_block=128, q_len=2048, causal=1, pooled_q=1, topk_num=1, topk_den=10,
                               n_first=1, n_last=1, dual_band=1, layout=p["layout"])
        idx, cnt, _, _ = bsa.bsa_select_blocks(qmean, kmean, sp, k_energy=ken, q_energy=qen)
        ap = bsa.attn_params(kv_block=128, q_block=128, cap=sp.cap, causal=1)
        o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap)
        o2, lse2, kept, _ = bsa.bsa_threshold_attention_fwd(qd, kd, vd, 1e-3)
        _sync()
        # entries of idx beyond cnt are documented as unwritten: compare the lists only
        valid = torch.arange(idx.shape[-1], device=idx.device) < cnt[..., None]
        idx = torch.where(valid, idx, torch.full_like(idx, -1))
        outs.append([t.clone() for t in (qmean, kmean, idx, cnt, o, lse, o2, lse2, kept)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_workspace_reuse(bsa):
    """One workspace serves many calls with identical results."""
    w = synth.dlm_denoise(L=2048 + 64, n_needles=2)
    p = w.params
    qd, kd, vd = _dev_workload(w)
    qprev = to_dev(w.extra["q_prev"], "bf16")
    mask, _ = bsa.bsa_active_rows(qd, qprev, p["theta_act"])
    kmean, _ = bsa.bsa_build_block_summaries(kd, 64, 0)
    sp = bsa.select_params(kv_block=64, q_block=32, q_pos0=p["q_pos0"], topk=16)
    ws_sel = torch.zeros(bsa.bsa_select_workspace_bytes(qd, 8, kmean.shape[2], sp), dtype=torch.uint8, device="cuda")
    wd = synth.gqa_decode(L=3000, n_needles=2)
    dq, dk, dv = _dev_workload(wd)
    dmean, _ = bsa.bsa_build_block_summaries(dk, 64, 0)
    dsp = bsa.select_params(kv_block=64, q_pos0=2999, topk=13, n_first=1, n_last=2, cap=16)
    didx, dcnt, _, _ = bsa.bsa_select_blocks(dq, dmean, dsp)
    dap = bsa.attn_params(kv_block=64, q_block=1, cap=16, q_pos0=2999)
    ws_att = torch.zeros(bsa.bsa_attention_workspace_bytes(dq, dk, dap), dtype=torch.uint8, device="cuda")
    ref = None
    for it in range(5):
        idx, cnt, _, _ = bsa.bsa_select_blocks(qd, kmean, sp, row_mask=mask, workspace=ws_sel)
        o, lse = bsa.bsa_sparse_attention_fwd(dq, dk, dv, didx, dcnt, dap, workspace=ws_att)
        _sync()
        valid = torch.arange(idx.shape[-1], device="cuda") < cnt[..., None]
        cur = (torch.where(valid, idx, -1).clone(), cnt.clone(), o.clone(), lse.clone())
        if ref is None:
            ref = cur
        else:
            assert all(torch.equal(a, b) for a, b in zip(ref, cur)), f"call {it} differs"


# ------------------------------------------------ ragged raw query blocks ---
def _raw_block_case(bsa, w, row_mask_np=None, stale_workspace=False):
    """Raw multi-row selection and attention on ``w`` (q_block from its params):
    lists against the oracle (tie band), then every unmasked row's output and
    LSE; rows with mask 0 must keep their cached values bit for bit.  With
    ``stale_workspace`` the selection runs on a workspace filled with 0xFF (as
    left by some other call), which must not leak into any list."""
    p = w.params
    qd, kd, vd = _dev_workload(w)
    B, Hq, Lq, D = qd.shape
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"])
    mask = None if row_mask_np is None else torch.from_numpy(row_mask_np.astype(np.uint8)).cuda()
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=p["q_block"], q_pos0=p["q_pos0"], causal=p["causal"],
                           topk=p["topk"], n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"],
                           scale=p["scale"], D=D)
    ws = None
    if stale_workspace:
        sp.cap = bsa.list_capacity(kmean.shape[2], min(p["q_block"], Lq), sp)
        ws = torch.full((bsa.bsa_select_workspace_bytes(qd, kd.shape[1], kmean.shape[2], sp),), 255,
                        dtype=torch.uint8, device="cuda")
    idx, cnt, rp, _ = bsa.bsa_select_blocks(qd, kmean, sp, row_mask=mask, want_row_picks=True, workspace=ws)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=p["q_block"], cap=sp.cap, q_pos0=p["q_pos0"],
                         causal=p["causal"], scale=p["scale"])
    cache_o = torch.randn(qd.shape, device="cuda")
    cache_l = torch.randn(qd.shape[:3], device="cuda")
    o, lse = bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx, cnt, ap, row_mask=mask, o=cache_o.clone(),
                                          lse=cache_l.clone())
    _sync()
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    km_ref, _ = orc.block_summaries(k, p["kv_block"], p["layout"])
    m_ref = None if row_mask_np is None else row_mask_np.astype(bool)
    sel = orc.select_blocks(p, km_ref, q=q, row_mask=m_ref)
    R = p["q_block"]
    idx_np, cnt_np, _ = _check_selection(sel, idx, cnt, rp, lambda qb: range(qb * R, min((qb + 1) * R, Lq)),
                                         w.name)
    O_ref, L_ref = orc.sparse_attention(p, q, k, v, _reference_lists(sel, idx_np, cnt_np), row_mask=m_ref)
    act = np.arange(Lq) if m_ref is None else np.nonzero(m_ref[0])[0]
    o_np, l_np = from_dev(o), lse.cpu().numpy()
    check_outputs(o_np[:, :, act], O_ref[:, :, act], l_np[:, :, act], L_ref[:, :, act], w.name)
    if m_ref is not None:
        stable = np.nonzero(~m_ref[0])[0]
        assert torch.equal(o[:, :, stable], cache_o[:, :, stable]), "a stable row's output was written"
        assert torch.equal(lse[:, :, stable], cache_l[:, :, stable]), "a stable row's LSE was written"
    return cnt_np


@pytest.mark.parametrize("Lq,masked,stale", [(33, False, False), (33, True, True), (65, True, False),
                                             (33, False, True)])
def test_select_one_row_last_block(bsa, Lq, masked, stale):
    """Lq % q_block == 1: the last query block has a single row and its list is that row's picks
    (raw rows, q_block 32), with and without a row mask, on a fresh or a stale workspace."""
    w = synth.dlm_denoise(L=2048 + 40, R=Lq, n_needles=3)
    w.params.update(q_block=32)
    mask = None
    if masked:
        rng = np.random.default_rng(Lq)
        mask = (rng.random((1, Lq)) < 0.4)
        mask[0, Lq - 1] = True                      # the one-row block is active
        mask[0, 0] = True
    cnt = _raw_block_case(bsa, w, mask, stale)
    assert cnt[0, :, -1].min() > 0


def test_select_one_row_last_block_masked_out(bsa):
    """The single row of the last query block is masked: its list is empty and the row keeps its cache."""
    w = synth.dlm_denoise(L=1024, R=33, n_needles=2)
    w.params.update(q_block=32)
    mask = np.ones((1, 33), dtype=bool)
    mask[0, 32] = False
    cnt = _raw_block_case(bsa, w, mask, True)
    assert (cnt[0, :, 1] == 0).all()


@pytest.mark.parametrize("q_pos0,Lq", [(4080, 64), (4090, 45), (4032, 64)])
def test_select_causal_raw_rows_unaligned(bsa, q_pos0, Lq):
    """Causal raw multi-row selection where query blocks straddle a KV-block edge: every candidate
    of a block (up to the block of its last row) is scored for every row of the block."""
    w = synth.dlm_denoise(L=4160, R=Lq, n_needles=3)
    w.params.update(q_block=32, q_pos0=q_pos0, causal=1)
    _raw_block_case(bsa, w)


@pytest.mark.parametrize("Hq,Hkv,R", [(16, 2, 32), (6, 2, 64), (8, 1, 48)])
def test_row_mask_direct_mfma_paths(bsa, Hq, Hkv, R):
    """Row masks on the direct (non-split) MFMA paths -- group size 8 with 32 rows, odd group size 3
    with 64 rows, group size 8 with 48 rows: stable rows keep their cached O and LSE bit for bit."""
    w = synth.dlm_denoise(L=2048 + 64, R=R, Hq=Hq, Hkv=Hkv, n_needles=2, n_active=R // 4)
    rng = np.random.default_rng(Hq * 100 + R)
    mask = rng.random((1, R)) < 0.5
    mask[0, 0] = True
    _raw_block_case(bsa, w, mask)


def test_select_exact_ties_take_lower_blocks(bsa):
    """21 copies of one needle block (bit-identical summaries, so equal scores in any precision)
    compete for 13 scored picks: the selection takes the 13 lowest block indices among them."""
    w = synth.gqa_decode(L=4096, Hq=8, Hkv=2, n_needles=1)
    p = w.params
    k = w.k.copy()
    copies = {}
    for g in range(2):
        nd = int(w.extra["needles"][g, 0])
        others = [j for j in range(1, 61) if j != nd][g * 3:g * 3 + 20]
        for j in others:
            k[0, g, 64 * j:64 * (j + 1)] = w.k[0, g, 64 * nd:64 * (nd + 1)]
        copies[g] = sorted(others + [nd])
    w.k = k
    qd, kd, vd = _dev_workload(w)
    kmean, _ = bsa.bsa_build_block_summaries(kd, 64, p["layout"])
    idx, cnt, rp, cap = _select_raw(bsa, w, qd, kmean)
    _sync()
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    NB = 64
    for g in range(2):
        got = set(idx_np[0, g, 0, :cnt_np[0, g, 0]].tolist())
        assert got == {0, NB - 2, NB - 1} | set(copies[g][:13]), (g, sorted(got))
    # the oracle agrees (its exact fp64 ties also go to the lower index)
    km_ref, _ = orc.block_summaries(w.f64("k"), 64, p["layout"])
    sel = orc.select_blocks(p, km_ref, q=w.f64("q"))
    for g in range(2):
        assert set(sel["lists"][0][g][0].tolist()) == {0, NB - 2, NB - 1} | set(copies[g][:13])
