"""bsa_denoise_step (active rows, their selection, prefix attention of the
active rows into the cache, block attention and merge, in three launches)
against the sequence of entry points it fuses and against the fp64 oracle.

Per sparse step, both paths start from the same prefix cache:
  * against bsa_active_rows + bsa_select_blocks(row_mask) +
    bsa_sparse_attention_fwd(row_mask, into the cache) +
    bsa_block_attention_merge: the row mask, the MSE and the list must be the
    same bits, and so must the rewritten cache and O / LSE (the same
    arithmetic in the same order, the list cut into the same slices);
  * against the oracle, carrying the oracle's own cache across the steps: the
    mask exactly, the union list within the 1e-6 tie band of the active rows'
    picks, O and LSE within the fp32 bounds on the lists the GPU chose.
Step 0 (every row, dense over the prefix) builds the cache with the separate
entry points, as the first denoising step of a block does."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from parity import ambiguous, check_list, check_outputs, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import dlm_bsa_block_amd as m
    m.lib()
    return m


def _sync():
    torch.cuda.synchronize()


def _select_params(bsa, p, R, D, causal=None):
    return bsa.select_params(kv_block=p["kv_block"], q_block=R, q_pos0=p["q_pos0"],
                             causal=p["causal"] if causal is None else causal, topk=p["topk"],
                             topk_num=p["topk_num"], topk_den=p["topk_den"], n_first=p["n_first"],
                             n_last=p["n_last"], layout=p["layout"], scale=p["scale"], D=D)


def _run_steps(bsa, w, theta=None, o_f32=True, causal=None, oracle=True, steps=None):
    p = w.params
    B, Hq, R, D = w.q.shape
    Hkv, L = w.k.shape[1], w.k.shape[2]
    theta = p["theta_act"] if theta is None else theta
    NB = -(-L // p["kv_block"])
    kd, vd = to_dev(w.k, "bf16"), to_dev(w.v, "bf16")
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"], with_energy=False)
    sp = _select_params(bsa, p, R, D, causal)
    sp.cap = bsa.list_capacity(NB, R, sp)
    causal = sp.causal
    cache_o = torch.zeros((B, Hq, R, D), device="cuda")
    cache_l = torch.zeros((B, Hq, R), device="cuda")
    qs = [to_dev(x, "bf16") for x in w.extra["q_steps"]]
    kbs = [to_dev(x, "bf16") for x in w.extra["kb_steps"]]
    vbs = [to_dev(x, "bf16") for x in w.extra["vb_steps"]]
    # step 0: every row, dense over the prefix, with the separate entry points
    idx0 = torch.arange(NB, dtype=torch.int32, device="cuda").view(1, 1, 1, NB).repeat(B, Hkv, 1, 1)
    cnt0 = torch.full((B, Hkv, 1), NB, dtype=torch.int32, device="cuda")
    ap0 = bsa.attn_params(kv_block=p["kv_block"], q_block=R, cap=NB, q_pos0=p["q_pos0"], causal=causal,
                          scale=p["scale"])
    bsa.bsa_sparse_attention_fwd(qs[0], kd, vd, idx0, cnt0, ap0, o=cache_o, lse=cache_l)
    if oracle:
        k64, v64 = w.f64("k"), w.f64("v")
        km_ref, _ = orc.block_summaries(k64, p["kv_block"], p["layout"])
        pr = dict(p, causal=causal)
        lists0 = [[[np.arange(NB)] for _ in range(Hkv)] for _ in range(B)]
        _, _, rO, rL = orc.denoise_step(pr, synth.storage_to_f64(w.extra["q_steps"][0], "bf16"), k64, v64,
                                        synth.storage_to_f64(w.extra["kb_steps"][0], "bf16"),
                                        synth.storage_to_f64(w.extra["vb_steps"][0], "bf16"), lists0, None,
                                        np.zeros((B, Hq, R, D)), np.zeros((B, Hq, R)))
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=R, cap=sp.cap, q_pos0=p["q_pos0"], causal=causal,
                         scale=p["scale"])
    ws = torch.empty(bsa.bsa_denoise_step_workspace_bytes(qs[0], kd, sp), dtype=torch.uint8, device="cuda")
    stats = []
    n = len(qs) if steps is None else steps
    for s in range(1, n):
        where = f"{w.name} step {s}"
        qd, qprev, kbd, vbd = qs[s], qs[s - 1], kbs[s], vbs[s]
        # the fused step
        fo, fl = cache_o.clone(), cache_l.clone()
        odt = torch.float32 if o_f32 else torch.bfloat16
        mask_f, mse_f, idx_f, cnt_f, o_f, l_f = bsa.bsa_denoise_step(
            qd, qprev, theta, kmean, kd, vd, kbd, vbd, sp, fo, fl, want_mse=True,
            o=torch.empty((B, Hq, R, D), dtype=odt, device="cuda"), workspace=ws)
        # the separate entry points
        mask_s, mse_s = bsa.bsa_active_rows(qd, qprev, theta)
        idx_s, cnt_s, _, _ = bsa.bsa_select_blocks(qd, kmean, sp, row_mask=mask_s)
        bsa.bsa_sparse_attention_fwd(qd, kd, vd, idx_s, cnt_s, ap, row_mask=mask_s, o=cache_o, lse=cache_l)
        o_s, l_s = bsa.bsa_block_attention_merge(qd, kbd, vbd, cache_o, cache_l, scale=p["scale"],
                                                 o=torch.empty((B, Hq, R, D), dtype=odt, device="cuda"))
        _sync()
        assert torch.equal(mask_f, mask_s), where + ": row mask"
        assert torch.equal(mse_f, mse_s), where + ": mse"
        assert torch.equal(cnt_f, cnt_s), where + ": list length"
        for b in range(B):
            for g in range(Hkv):
                c = int(cnt_s[b, g, 0])
                assert torch.equal(idx_f[b, g, 0, :c], idx_s[b, g, 0, :c]), f"{where}: list b{b} g{g}"
        assert torch.equal(fo, cache_o) and torch.equal(fl, cache_l), where + ": prefix cache"
        assert torch.equal(o_f, o_s) and torch.equal(l_f, l_s), where + ": output"
        n_act = int(mask_f.sum().item())
        stats.append(dict(active=n_act, list_blocks=cnt_f[0, :, 0].cpu().tolist()))
        if oracle:
            q64 = synth.storage_to_f64(w.extra["q_steps"][s], "bf16")
            kb64 = synth.storage_to_f64(w.extra["kb_steps"][s], "bf16")
            vb64 = synth.storage_to_f64(w.extra["vb_steps"][s], "bf16")
            m_ref, mse_ref = orc.active_rows(q64, synth.storage_to_f64(w.extra["q_steps"][s - 1], "bf16"), theta)
            assert np.array_equal(mask_f.cpu().numpy().astype(bool), m_ref), where + ": mask vs oracle"
            sel = orc.select_blocks(pr, km_ref, q=q64, row_mask=m_ref)
            idx_np, cnt_np = idx_f.cpu().numpy(), cnt_f.cpu().numpy()
            lists = [[[None] for _ in range(Hkv)] for _ in range(B)]
            for b in range(B):
                for g in range(Hkv):
                    band = set()
                    for r in range(R):
                        if (b, g, r) in sel["rows"]:
                            band |= ambiguous(sel["rows"][(b, g, r)])
                    ol = sel["lists"][b][g][0]
                    check_list(idx_np[b, g, 0], int(cnt_np[b, g, 0]), ol, band, f"{where} b{b} g{g}")
                    gl = idx_np[b, g, 0, :cnt_np[b, g, 0]].astype(np.int64)
                    lists[b][g][0] = ol if np.array_equal(gl, ol) else gl
            O_ref, L_ref, rO, rL = orc.denoise_step(pr, q64, k64, v64, kb64, vb64, lists, m_ref, rO, rL)
            if o_f32:
                check_outputs(from_dev(o_f), O_ref, l_f.cpu().numpy(), L_ref, where)
            check_outputs(from_dev(fo), rO, fl.cpu().numpy(), rL, where + " (prefix cache)")
    return stats


def test_denoise_step_small(bsa):
    """Four steps over a 2152-token prefix (34 blocks, the last ragged), 4 rows change per step."""
    w = synth.dlm_denoise_steps(L=2048 + 64 + 40, n_needles=2, n_steps=4)
    st = _run_steps(bsa, w)
    assert all(x["active"] == 4 for x in st)


def _stack(wa, wb):
    """Two denoising workloads of the same shapes as one of batch 2."""
    cat = lambda x, y: np.concatenate([x, y], axis=0)
    extra = dict(q_steps=[cat(x, y) for x, y in zip(wa.extra["q_steps"], wb.extra["q_steps"])],
                 kb_steps=[cat(x, y) for x, y in zip(wa.extra["kb_steps"], wb.extra["kb_steps"])],
                 vb_steps=[cat(x, y) for x, y in zip(wa.extra["vb_steps"], wb.extra["vb_steps"])])
    return synth.Workload("dlm_denoise_steps_b2", wa.dtype, cat(wa.q, wb.q), cat(wa.k, wb.k), cat(wa.v, wb.v),
                          dict(wa.params), extra)


def test_denoise_step_batch_two(bsa):
    """Two sequences in one call: different prefixes, queries and active rows per batch entry."""
    w = _stack(synth.dlm_denoise_steps(seed=6, L=1024 + 64 + 5, n_needles=2, n_steps=3),
               synth.dlm_denoise_steps(seed=9, L=1024 + 64 + 5, n_needles=2, n_steps=3))
    st = _run_steps(bsa, w)
    assert all(x["active"] == 8 for x in st)


def test_denoise_step_bf16_out_causal(bsa):
    """bf16 output and the causal flag (the prefix lies before the block: every key stays visible)."""
    w = synth.dlm_denoise_steps(L=1024 + 64 + 3, n_needles=2, n_steps=3)
    _run_steps(bsa, w, o_f32=False, causal=1)


@pytest.mark.parametrize("R,Hq,Hkv", [(20, 16, 4), (16, 16, 2), (9, 8, 8)])
def test_denoise_step_short_block(bsa, R, Hq, Hkv):
    """Blocks of fewer rows than the 32-row tiles (a ragged combine chunk for R = 9); group sizes 4, 8, 1."""
    w = synth.dlm_denoise_steps(L=1024 + 7, R=R, Hq=Hq, Hkv=Hkv, n_needles=2, n_steps=3, per_step=3)
    st = _run_steps(bsa, w)
    assert all(x["active"] == 3 for x in st)


def test_denoise_step_every_row_active(bsa):
    """theta below every MSE: all rows recompute (the union of all picks, several slices per workgroup)."""
    w = synth.dlm_denoise_steps(L=4096 + 64, n_needles=2, n_steps=2)
    st = _run_steps(bsa, w, theta=-1.0)
    assert st[0]["active"] == 32


def test_denoise_step_no_active_rows(bsa):
    """theta above every MSE: no row recomputes, the lists are empty, the cache keeps its bits and every
    row still merges its cached prefix with the block's own keys."""
    w = synth.dlm_denoise_steps(L=1024 + 64, n_needles=2, n_steps=2)
    st = _run_steps(bsa, w, theta=1e30)
    assert st[0]["active"] == 0 and all(c == 0 for c in st[0]["list_blocks"])


def test_denoise_step_full_size(bsa):
    """The benchmark's 32K prefix: three sparse steps, checked bit for bit against the separate entry
    points and against the oracle."""
    w = synth.dlm_denoise_steps(n_steps=4)
    st = _run_steps(bsa, w)
    assert all(max(x["list_blocks"]) < 512 for x in st)


def test_denoise_step_rejects(bsa):
    """Shapes outside the fused step fail with an error, before any launch."""
    w = synth.dlm_denoise_steps(L=1024, n_needles=1, n_steps=2)
    p = w.params
    B, Hq, R, D = w.q.shape
    kd, vd = to_dev(w.k, "bf16"), to_dev(w.v, "bf16")
    kmean, _ = bsa.bsa_build_block_summaries(kd, p["kv_block"], p["layout"], with_energy=False)
    q = to_dev(w.extra["q_steps"][1], "bf16")
    kb, vb = to_dev(w.extra["kb_steps"][1], "bf16"), to_dev(w.extra["vb_steps"][1], "bf16")
    co, cl = torch.zeros((B, Hq, R, D), device="cuda"), torch.zeros((B, Hq, R), device="cuda")
    sp = _select_params(bsa, p, R, D)
    bad_q = _select_params(bsa, p, R // 2, D)                        # q_block != R
    with pytest.raises(bsa.BsaError):
        bsa.bsa_denoise_step(q, q, 0.1, kmean, kd, vd, kb, vb, bad_q, co, cl)
    with pytest.raises(bsa.BsaError):                                # a bf16 cache
        bsa.bsa_denoise_step(q, q, 0.1, kmean, kd, vd, kb, vb, sp, co.to(torch.bfloat16), cl)
    with pytest.raises(bsa.BsaError):                                # a non-finite theta
        bsa.bsa_denoise_step(q, q, float("nan"), kmean, kd, vd, kb, vb, sp, co, cl)
