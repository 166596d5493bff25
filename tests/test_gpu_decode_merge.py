"""Decode attention (single-row query blocks) with its split-KV slices merged
inside the attention launch -- up to 1024 (batch, KV head, row) triples, the
last workgroup of a row to finish merges -- and with the separate combine
launch beyond that.  Both are compared with the oracle on given block lists,
including empty lists (O = 0, LSE = -inf) and a row mask (stable rows keep
their cached values).  One zeroed workspace reused across shapes and both
paths must give the bits a fresh workspace gives."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from checks import check_outputs
from parity import from_dev, to_dev

pytestmark = pytest.mark.gpu

ROWS_MERGED_MAX = 1024      # (batch, KV head, row) triples the in-launch merge counts


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import dlm_bsa_block_amd as m
    m.lib()
    return m


def _run(bsa, w, row_mask=None, ws=None, f32_out=True):
    p = w.params
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    idx = torch.from_numpy(w.extra["idx"]).cuda()
    cnt = torch.from_numpy(w.extra["cnt"]).cuda()
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=p["cap"], q_pos0=p["q_pos0"], scale=p["scale"])
    odt = torch.float32 if f32_out else torch.bfloat16
    o0 = torch.full(q.shape, 7.0, dtype=odt, device="cuda")
    l0 = torch.full(q.shape[:3], 7.0, dtype=torch.float32, device="cuda")
    rm = None if row_mask is None else torch.from_numpy(row_mask).cuda()
    o, lse = bsa.bsa_sparse_attention_fwd(q, k, v, idx, cnt, ap, row_mask=rm, o=o0, lse=l0, workspace=ws)
    torch.cuda.synchronize()
    return o, lse, bsa.bsa_attention_workspace_bytes(q, k, ap)


def _check(w, o, lse, row_mask=None, heads=(0, 5, 13, 31)):
    p = dict(w.params, causal=0)
    lists = [[[w.extra["idx"][0, g, r, :w.extra["cnt"][0, g, r]].astype(np.int64)
               for r in range(w.q.shape[2])] for g in range(w.k.shape[1])]]
    O_ref, L_ref = orc.sparse_attention(p, w.f64("q"), w.f64("k"), w.f64("v"), lists, row_mask=row_mask,
                                        heads=list(heads))
    og, lg = from_dev(o), from_dev(lse)
    rows = np.arange(w.q.shape[2]) if row_mask is None else np.nonzero(row_mask[0])[0]
    hs = list(heads)
    check_outputs(og[:, hs][:, :, rows], O_ref[:, hs][:, :, rows], lg[:, hs][:, :, rows], L_ref[:, hs][:, :, rows],
                  w.name)
    if row_mask is not None:                     # stable rows: untouched, every head
        stable = np.nonzero(row_mask[0] == 0)[0]
        assert (og[:, :, stable] == 7.0).all() and (lg[:, :, stable] == 7.0).all()
    # empty lists: O = 0 and LSE = -inf, every head of the group
    for g in range(w.k.shape[1]):
        G = w.q.shape[1] // w.k.shape[1]
        for r in np.nonzero(w.extra["cnt"][0, g] == 0)[0]:
            if row_mask is not None and row_mask[0, r] == 0:
                continue
            assert (og[0, g * G:(g + 1) * G, r] == 0).all() and np.isneginf(lg[0, g * G:(g + 1) * G, r]).all()


@pytest.mark.parametrize("Lq", [1, 37, 128])
def test_merged_in_launch(bsa, Lq):
    """8 KV heads x Lq rows <= 1024: the slices merge in the attention launch."""
    w = synth.decode_rows(Lq=Lq, L=4096 if Lq > 1 else 6000)
    assert 8 * Lq <= ROWS_MERGED_MAX
    o, lse, _ = _run(bsa, w)
    _check(w, o, lse)


def test_merged_bf16_is_rounded_f32(bsa):
    w = synth.decode_rows(Lq=16, L=3000, seed=8)
    o32, l32, _ = _run(bsa, w)
    o16, l16, _ = _run(bsa, w, f32_out=False)
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(l16, l32)


def test_combine_beyond_counter_region(bsa):
    """8 KV heads x 129 rows = 1032 > 1024 triples: the separate combine runs."""
    w = synth.decode_rows(Lq=129, L=4096, seed=9)
    o, lse, _ = _run(bsa, w)
    _check(w, o, lse)


@pytest.mark.parametrize("Lq", [40, 130])
def test_row_mask(bsa, Lq):
    w = synth.decode_rows(Lq=Lq, L=4096, seed=10)
    rm = np.zeros((1, Lq), dtype=np.uint8)
    rm[0, ::3] = 1
    o, lse, _ = _run(bsa, w, row_mask=rm)
    _check(w, o, lse, row_mask=rm)


def test_workspace_reused_across_shapes(bsa):
    """One zeroed workspace, sized for the largest call, serves merged and
    combined decodes of several shapes in turn: each result equals, bit for
    bit, the one a fresh zeroed workspace gives."""
    ws_ = [synth.decode_rows(Lq=Lq, L=L, seed=s) for Lq, L, s in ((8, 3000, 11), (140, 4096, 12), (64, 5000, 13))]
    fresh = [_run(bsa, w) for w in ws_]
    need = max(f[2] for f in fresh)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for w, (o_f, l_f, _) in zip(ws_, fresh):
            o, lse, _ = _run(bsa, w, ws=ws)
            assert torch.equal(o, o_f) and torch.equal(lse, l_f), f"{w.name} Lq={w.q.shape[2]} rep {rep}"
    # the counters are back to zero after every call
    assert not ws[:65536].any()


@pytest.mark.parametrize("Lq,window", [(40, 300), (130, 700)])
def test_window_merged_and_combined(bsa, Lq, window):
    """Selected blocks plus a sliding window (two branches mixed by gates),
    merged in the launch (8 x 40 triples) and by the combine (8 x 130), both
    against the oracle's two branches."""
    w = synth.decode_rows(Lq=Lq, L=4096, seed=14)
    p = w.params
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    idx = torch.from_numpy(w.extra["idx"]).cuda()
    cnt = torch.from_numpy(w.extra["cnt"]).cuda()
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=p["cap"], q_pos0=p["q_pos0"], scale=p["scale"])
    gates = np.random.default_rng(Lq).uniform(0.1, 1.2, (1, q.shape[1], Lq, 2)).astype(np.float32)
    o, lse = bsa.bsa_window_decode_fwd(q, k, v, idx, cnt, ap, window, gates=torch.from_numpy(gates).cuda(),
                                       o=torch.zeros(q.shape, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    lists = [[[w.extra["idx"][0, g, r, :w.extra["cnt"][0, g, r]].astype(np.int64) for r in range(Lq)]
              for g in range(w.k.shape[1])]]
    O_ref, L_ref = orc.window_decode(dict(p, causal=0), w.f64("q"), w.f64("k"), w.f64("v"), lists, window,
                                     gates.astype(np.float64))
    check_outputs(from_dev(o), O_ref, lse.cpu().numpy(), L_ref, f"window {window} Lq {Lq}")


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (16, 8, 128), (32, 4, 128), (32, 8, 64)])
def test_merged_group_sizes(bsa, Hq, Hkv, D):
    """Group sizes 1, 2 and 8 (8: two (head, dim pair) positions per thread in
    the merge) and head dim 64, merged in the launch."""
    w = synth.decode_rows(Lq=20, L=3000, Hq=Hq, Hkv=Hkv, D=D, seed=15)
    o, lse, _ = _run(bsa, w)
    _check(w, o, lse, heads=tuple(sorted({0, Hq // 2 - 1, Hq - 1})))


@pytest.mark.parametrize("Lq", [40, 70])
def test_batch_two(bsa, Lq):
    """Two batch entries (2 x 8 x 40 triples merged in the launch, 2 x 8 x 70
    past the counter region), each against the oracle on its own lists."""
    ws_ = [synth.decode_rows(Lq=Lq, L=3500, seed=s) for s in (16, 17)]
    p = ws_[0].params
    cat = lambda name: np.concatenate([getattr(x, name) for x in ws_])
    q, k, v = (to_dev(cat(n), "bf16") for n in ("q", "k", "v"))
    idx = torch.from_numpy(np.concatenate([x.extra["idx"] for x in ws_])).cuda()
    cnt = torch.from_numpy(np.concatenate([x.extra["cnt"] for x in ws_])).cuda()
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=p["cap"], q_pos0=p["q_pos0"], scale=p["scale"])
    o, lse = bsa.bsa_sparse_attention_fwd(q, k, v, idx, cnt, ap,
                                          o=torch.zeros(q.shape, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    og, lg = from_dev(o), from_dev(lse)
    for b, w in enumerate(ws_):
        heads = [0, 9, 22, 31]
        lists = [[[w.extra["idx"][0, g, r, :w.extra["cnt"][0, g, r]].astype(np.int64) for r in range(Lq)]
                  for g in range(w.k.shape[1])]]
        O_ref, L_ref = orc.sparse_attention(dict(p, causal=0), w.f64("q"), w.f64("k"), w.f64("v"), lists,
                                            heads=heads)
        check_outputs(og[b:b + 1, heads], O_ref[:, heads], lg[b:b + 1, heads], L_ref[:, heads], f"batch {b}")


def test_repeated_calls_are_bitwise_equal(bsa):
    """300 calls on one workspace, alternating a merged and a combined shape, at
    the full 64K-like slice count per row (32 slices): every result equals the
    first bit for bit.  A merge that read a partial before it was published
    would differ from run to run."""
    shapes = [synth.decode_rows(Lq=Lq, L=8192, seed=s) for Lq, s in ((4, 18), (130, 19))]
    args = []
    for w in shapes:
        p = w.params
        q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
        idx = torch.from_numpy(w.extra["idx"]).cuda()
        cnt = torch.from_numpy(w.extra["cnt"]).cuda()
        ap = bsa.attn_params(kv_block=p["kv_block"], q_block=1, cap=p["cap"], q_pos0=p["q_pos0"], scale=p["scale"])
        args.append((q, k, v, idx, cnt, ap))
    need = max(bsa.bsa_attention_workspace_bytes(a[0], a[1], a[5]) for a in args)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = [bsa.bsa_sparse_attention_fwd(*a, workspace=ws) for a in args]
    first = [(o.clone(), l.clone()) for o, l in first]
    for it in range(300):
        o, lse = bsa.bsa_sparse_attention_fwd(*args[it % 2], workspace=ws)
        if it % 50 == 49 or it < 2:
            torch.cuda.synchronize()
        assert torch.equal(o, first[it % 2][0]) and torch.equal(lse, first[it % 2][1]), f"call {it}"
    torch.cuda.synchronize()
    assert not ws[:65536].any()
