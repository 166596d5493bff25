"""bsa_decode_step (selection with the newest block's summary refresh, then
attention over the selected blocks, in two launches) against the fp64
oracle, and against the separate entry points it combines.

Per case: the refreshed summary (mean and band energies) against the oracle's
summaries and bit for bit against the separate refresh; the lists with the 1e-6 tie band; O and LSE against the oracle on
the lists the GPU chose (outside the tie band they are the oracle's).  Where
the fused step and bsa_select_blocks_refresh + bsa_sparse_attention_fwd chose
the same list, their outputs must be the same bits when both attend in the
same form (the attention arithmetic is shared; only the selection's
normalisers are summed in another order): f32 or D = 64 lists, and the
lengthened slices of many lists; a single bf16 row with D = 128 is attended on
the matrix cores by the entry point and with vector products by the step, and
both are checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from parity import check_list, check_outputs, from_dev, to_dev, ambiguous

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import dlm_bsa_block_amd as m
    m.lib()
    return m


def _step_case(bsa, w, refresh=True, odtype=None):
    p = w.params
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    B, Hq, Lq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    NB = -(-L // p["kv_block"])
    kmean, kenergy = bsa.bsa_build_block_summaries(k, p["kv_block"], p["layout"])
    rb = NB - 1 if refresh else -1
    if refresh:
        kmean[:, :, rb] = 0.0          # stale: the step must pool it again
        kenergy[:, :, rb] = 0.0
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=1, q_pos0=p["q_pos0"], causal=p["causal"],
                           topk=p["topk"], topk_num=p.get("topk_num", 0), topk_den=p.get("topk_den", 1),
                           n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"], scale=p["scale"], D=D)
    km2, ke2 = kmean.clone(), kenergy.clone()
    o = torch.empty(q.shape, dtype=q.dtype if odtype is None else odtype, device="cuda")
    idx, cnt, o, lse = bsa.bsa_decode_step(q, k, v, kmean, sp, refresh_block=rb, k_energy=kenergy, o=o)
    # the same step through the separate entry points
    sp2 = bsa.select_params(kv_block=p["kv_block"], q_block=1, q_pos0=p["q_pos0"], causal=p["causal"],
                            topk=p["topk"], topk_num=p.get("topk_num", 0), topk_den=p.get("topk_den", 1),
                            n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"], scale=p["scale"], D=D,
                            cap=sp.cap)
    if refresh:
        idx2, cnt2, _ = bsa.bsa_select_blocks_refresh(k, rb, q, km2, sp2, k_energy=ke2)
    else:
        idx2, cnt2, _, _ = bsa.bsa_select_blocks(q, km2, sp2)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=sp.cap, q_pos0=p["q_pos0"], causal=p["causal"],
                         scale=p["scale"], D=D)
    o2, lse2 = bsa.bsa_sparse_attention_fwd(q, k, v, idx2, cnt2, ap, o=torch.empty_like(o))
    torch.cuda.synchronize()
    qf, kf, vf = w.f64("q"), w.f64("k"), w.f64("v")
    km_ref, ke_ref = orc.block_summaries(kf, p["kv_block"], p["layout"])
    if refresh:
        assert np.allclose(from_dev(kmean[:, :, rb]), km_ref[:, :, rb], rtol=1e-5, atol=2e-6)
        assert np.allclose(from_dev(kenergy[:, :, rb]), ke_ref[:, :, rb], rtol=1e-5, atol=1e-5)
        assert torch.equal(kmean[:, :, :rb], km2[:, :, :rb])        # nothing else written
        # pooled in the block-summary kernel's fixed order, as the separate refresh: the same bits
        assert torch.equal(kmean, km2) and torch.equal(kenergy, ke2)
    sel = orc.select_blocks(p, km_ref, q=qf)
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    idx2_np, cnt2_np = idx2.cpu().numpy(), cnt2.cpu().numpy()
    lists = [[[None] * Lq for _ in range(Hkv)] for _ in range(B)]
    same = np.ones((B, Hkv, Lq), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for r in range(Lq):
                band = ambiguous(sel["rows"][(b, g, r)])
                check_list(idx_np[b, g, r], int(cnt_np[b, g, r]), sel["lists"][b][g][r], band,
                           f"{w.name} step b{b} g{g} r{r}")
                gl = idx_np[b, g, r, :cnt_np[b, g, r]].astype(np.int64)
                lists[b][g][r] = gl
                same[b, g, r] = cnt_np[b, g, r] == cnt2_np[b, g, r] and np.array_equal(
                    gl, idx2_np[b, g, r, :cnt2_np[b, g, r]])
    O_ref, L_ref = orc.sparse_attention(p, qf, kf, vf, lists)
    if o.dtype == torch.float32:
        stats = check_outputs(from_dev(o), O_ref, lse.cpu().numpy(), L_ref, f"{w.name} step")
    else:
        # bf16 output: compare the f32 run of the same step, then the rounding
        o32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        _, _, o32, lse32 = bsa.bsa_decode_step(q, k, v, kmean, sp, refresh_block=rb, k_energy=kenergy, o=o32)
        torch.cuda.synchronize()
        stats = check_outputs(from_dev(o32), O_ref, lse32.cpu().numpy(), L_ref, f"{w.name} step")
        assert torch.equal(o.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
        assert torch.equal(lse, lse32)
    G = Hq // Hkv
    # bf16 lists with D = 128 on 32-token slices: the entry point scores on the matrix cores, the
    # step with vector products (another summation order); both against the oracle then
    same_form = not (w.dtype == "bf16" and D == 128)
    if not same_form:
        lists2 = [[[idx2_np[b, g, r, :cnt2_np[b, g, r]].astype(np.int64) for r in range(Lq)] for g in range(Hkv)]
                  for b in range(B)]
        O_ref2, L_ref2 = orc.sparse_attention(p, qf, kf, vf, lists2)
        check_outputs(from_dev(o2), O_ref2, lse2.cpu().numpy(), L_ref2, f"{w.name} entry point")
    for b in range(B):
        for g in range(Hkv):
            for r in range(Lq):
                if same[b, g, r] and same_form:
                    hs = slice(g * G, (g + 1) * G)
                    assert torch.equal(o[b, hs, r], o2[b, hs, r]), (b, g, r)
                    assert torch.equal(lse[b, hs, r], lse2[b, hs, r]), (b, g, r)
    assert same.mean() > 0.5
    return idx_np, cnt_np, stats


@pytest.mark.parametrize("L", [8192, 8000, 1000])
def test_decode_step_small(bsa, L):
    w = synth.gqa_decode(L=L, n_needles=4)
    idx, cnt, _ = _step_case(bsa, w)
    NB = -(-L // 64)
    for g in range(8):
        lst = set(idx[0, g, 0, :cnt[0, g, 0]].tolist())
        assert len(lst) == 16 and {0, NB - 2, NB - 1} <= lst
        assert set(w.extra["needles"][g].tolist()) <= lst


def test_decode_step_full_size(bsa):
    """64K decode, 32 query / 8 KV heads: the benchmark's workload and launch."""
    w = synth.gqa_decode()
    idx, cnt, _ = _step_case(bsa, w)
    assert (cnt == 16).all()


def test_decode_step_no_refresh_f32_out(bsa):
    w = synth.gqa_decode(L=4096 + 37, n_needles=3)
    _step_case(bsa, w, refresh=False, odtype=torch.float32)


def test_decode_step_tiny_f32(bsa):
    """fp32 inputs, head dim 64, one head, 16 blocks of which 4 are kept."""
    idx, cnt, _ = _step_case(bsa, synth.tiny_decode())
    assert cnt[0, 0, 0] == 4 and {0, 15} <= set(idx[0, 0, 0, :4].tolist())


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 1, 128), (4, 2, 64), (6, 6, 128)])
def test_decode_step_group_sizes(bsa, Hq, Hkv, D):
    w = synth.gqa_decode(L=3000, Hq=Hq, Hkv=Hkv, D=D, n_needles=3)
    _step_case(bsa, w)


def test_decode_step_rows_causal(bsa):
    """Three decode rows at positions L-3 .. L-1 with causal masking: each row has its own candidates
    (the newest block is visible to the last rows only when it starts before them)."""
    w = synth.gqa_decode(L=4096 + 2, Hq=8, Hkv=2, n_needles=3)
    qpos = w.params["q_pos0"]
    # rows: the stored query repeated at three positions with small seeded offsets
    rng = np.random.default_rng(11)
    q = synth.storage_to_f64(w.q, "bf16")
    q3 = np.concatenate([q, q + 0.3 * rng.standard_normal(q.shape), q - 0.2 * rng.standard_normal(q.shape)], axis=2)
    w.q = synth.f32_to_bf16_bits(q3.astype(np.float32))
    w.params.update(q_pos0=qpos - 2, causal=1)
    idx, cnt, _ = _step_case(bsa, w, refresh=False)
    NB = 65
    # row 0 sits at 4095, before the last block (keys 4096, 4097); rows 1 and 2 see it
    for g in range(2):
        assert (idx[0, g, 0, :cnt[0, g, 0]] < NB - 1).all()
        assert NB - 1 in idx[0, g, 1, :cnt[0, g, 1]] and NB - 1 in idx[0, g, 2, :cnt[0, g, 2]]


def test_decode_step_many_blocks(bsa):
    """More than 1024 blocks (the wide selection path): 1500 blocks of 64."""
    w = synth.gqa_decode(L=64 * 1500 - 5, Hq=8, Hkv=2, n_needles=6)
    idx, cnt, _ = _step_case(bsa, w)
    assert (cnt == 16).all()


def test_decode_step_fractional_budget(bsa):
    """k' = ceil(0.05 * |C|) scored picks instead of a fixed count."""
    w = synth.gqa_decode(L=9000, Hq=8, Hkv=2, n_needles=3)
    w.params.update(topk=0, topk_num=1, topk_den=20)
    idx, cnt, _ = _step_case(bsa, w)
    NB = -(-9000 // 64)
    assert (cnt == min(NB, 3 + -(-NB // 20))).all()


def test_decode_step_shifted_batch_full_size(bsa):
    """32 sequences of 64K in one call (the batched decode measurement's inputs
    and launch): sequence b is the 64K cache rolled by synth.decode_batch_shifts.
    Sampled sequences against the oracle (refreshed summary, lists with the tie
    band, O and LSE); the attention entry point on the step's lists, at batch
    32 (lengthened slices, scores on the matrix cores) and on the first 4
    (32-token slices), against the oracle on the same lists.  At batch 32 the
    step and the entry point share slices and arithmetic: the same bits."""
    w = synth.gqa_decode()
    p = w.params
    B = 32
    q1, k1, v1 = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    _, Hkv, L, D = k1.shape
    shifts = synth.decode_batch_shifts(B, L, p["kv_block"])
    k = torch.empty((B, Hkv, L, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    for b, sh in enumerate(shifts):
        k[b].copy_(torch.roll(k1[0], sh, dims=1))
        v[b].copy_(torch.roll(v1[0], sh, dims=1))
    del k1, v1
    q = q1.expand(B, -1, -1, -1).contiguous()
    NB = L // p["kv_block"]
    kmean, kenergy = bsa.bsa_build_block_summaries(k, p["kv_block"], p["layout"])
    kmean[:, :, NB - 1] = 0.0                  # stale: the step pools it again
    kenergy[:, :, NB - 1] = 0.0
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=1, q_pos0=p["q_pos0"], topk=p["topk"],
                           n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"], scale=p["scale"])
    idx, cnt, o, lse = bsa.bsa_decode_step(q, k, v, kmean, sp, refresh_block=NB - 1, k_energy=kenergy)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=sp.cap, q_pos0=p["q_pos0"], scale=p["scale"])
    o2, lse2 = bsa.bsa_sparse_attention_fwd(q, k, v, idx, cnt, ap)
    o4, lse4 = bsa.bsa_sparse_attention_fwd(q[:4], k[:4], v[:4], idx[:4], cnt[:4], ap)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    assert (cnt_np == 16).all()
    # distinct sequences select distinct lists
    assert len({tuple(idx_np[b, 0, 0, :16].tolist()) for b in range(B)}) > B // 2
    qf = w.f64("q")
    for b in (0, 1, 17, B - 1):
        print(f"shifted batch: oracle for sequence {b} (shift {shifts[b]})", flush=True)
        kf = synth.storage_to_f64(synth.shift_sequence(w.k[0], shifts[b]), "bf16")[None]
        vf = synth.storage_to_f64(synth.shift_sequence(w.v[0], shifts[b]), "bf16")[None]
        km_ref, ke_ref = orc.block_summaries(kf, p["kv_block"], p["layout"])
        assert np.allclose(from_dev(kmean[b, :, NB - 1]), km_ref[0, :, NB - 1], rtol=1e-5, atol=2e-6)
        assert np.allclose(from_dev(kenergy[b, :, NB - 1]), ke_ref[0, :, NB - 1], rtol=1e-5, atol=1e-5)
        sel = orc.select_blocks(p, km_ref, q=qf)
        lists = [[[None] for _ in range(Hkv)]]
        for g in range(Hkv):
            band = ambiguous(sel["rows"][(0, g, 0)])
            check_list(idx_np[b, g, 0], int(cnt_np[b, g, 0]), sel["lists"][0][g][0], band,
                       f"shifted batch b{b} g{g}")
            lists[0][g][0] = idx_np[b, g, 0, :cnt_np[b, g, 0]].astype(np.int64)
        O_ref, L_ref = orc.sparse_attention(p, qf, kf, vf, lists)
        check_outputs(from_dev(o[b:b + 1]), O_ref, lse[b:b + 1].cpu().numpy(), L_ref, f"shifted batch b{b}")
        check_outputs(from_dev(o2[b:b + 1]), O_ref, lse2[b:b + 1].cpu().numpy(), L_ref, f"entry point, b{b}")
        if b < 4:
            check_outputs(from_dev(o4[b:b + 1]), O_ref, lse4[b:b + 1].cpu().numpy(), L_ref, f"batch of 4, b{b}")
        del kf, vf
