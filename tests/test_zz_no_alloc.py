"""bsa_sparse_attention_fwd_noalloc: the attention entry point that takes no
workspace (its arrival counters and split-KV partials live in the library's static device scratch).
Two calls in a row through the C ABI -- a denoising block (32 rows, split MFMA
path) and then a smaller decode step -- each equal, bit for bit, to
bsa_sparse_attention_fwd with a caller workspace on the same inputs; the
scratch keeps the first call's contents when the second runs."""
import numpy as np
import pytest
import torch

import synth
from parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import dlm_bsa_block_amd as m
    m.lib()
    return m


def _inputs(bsa, w, row_mask=None):
    p = w.params
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    kmean, _ = bsa.bsa_build_block_summaries(k, p["kv_block"], p["layout"])
    sp = bsa.select_params(kv_block=p["kv_block"], q_block=p["q_block"], q_pos0=p["q_pos0"], topk=p["topk"],
                           n_first=p["n_first"], n_last=p["n_last"], layout=p["layout"], scale=p["scale"],
                           D=q.shape[3])
    idx, cnt, _, _ = bsa.bsa_select_blocks(q, kmean, sp, row_mask=row_mask)
    ap = bsa.attn_params(kv_block=p["kv_block"], q_block=p["q_block"], cap=sp.cap, q_pos0=p["q_pos0"],
                         scale=p["scale"], D=q.shape[3])
    return q, k, v, idx, cnt, ap


def _compare(bsa, q, k, v, idx, cnt, ap, row_mask=None, odtype=None):
    odtype = q.dtype if odtype is None else odtype
    base_o = torch.randn(q.shape, device="cuda").to(odtype)
    base_l = torch.randn(q.shape[:3], device="cuda")
    ws = torch.zeros(max(256, bsa.bsa_attention_workspace_bytes(q, k, ap)), dtype=torch.uint8, device="cuda")
    o_ref, l_ref = bsa.bsa_sparse_attention_fwd(q, k, v, idx, cnt, ap, row_mask=row_mask, o=base_o.clone(),
                                                lse=base_l.clone(), workspace=ws)
    o, lse = bsa.bsa_sparse_attention_fwd_noalloc(q, k, v, idx, cnt, ap, base_o.clone(), base_l.clone(),
                                                  row_mask=row_mask)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                       o_ref.view(torch.int16) if o_ref.dtype == torch.bfloat16 else o_ref)
    assert torch.equal(lse, l_ref)
    assert torch.isfinite(o.float()).all()


def test_noalloc_two_calls_second_smaller(bsa):
    assert bsa.lib().bsa_noalloc_scratch_bytes() == 64 << 20
    # first call: a 32-row denoising block over a 4K prefix, 8 active rows (split MFMA path + combine)
    w1 = synth.dlm_denoise(L=4096 + 64, n_needles=3)
    mask = torch.zeros((1, 32), dtype=torch.uint8, device="cuda")
    mask[0, w1.extra["active"]] = 1
    q, k, v, idx, cnt, ap = _inputs(bsa, w1, mask)
    need1 = bsa.bsa_attention_workspace_bytes(q, k, ap)
    _compare(bsa, q, k, v, idx, cnt, ap, row_mask=mask, odtype=torch.float32)
    # second call: a smaller decode step (VALU split-KV path + combine), bf16 and f32 outputs
    w2 = synth.gqa_decode(L=2048 + 37, Hq=8, Hkv=2, n_needles=2)
    q2, k2, v2, idx2, cnt2, ap2 = _inputs(bsa, w2)
    need2 = bsa.bsa_attention_workspace_bytes(q2, k2, ap2)
    assert 0 < need2 < need1
    _compare(bsa, q2, k2, v2, idx2, cnt2, ap2)
    _compare(bsa, q2, k2, v2, idx2, cnt2, ap2, odtype=torch.float32)


def test_noalloc_rejects_oversized_scratch(bsa):
    """A call that would need more than the static scratch is rejected before anything runs."""
    q = torch.empty((1, 32, 64 * 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((1, 8, 64, 4096), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, 8, 64), dtype=torch.int32, device="cuda")
    ap = bsa.attn_params(kv_block=64, q_block=32, cap=4096)
    assert bsa.bsa_attention_workspace_bytes(q, k, ap) > bsa.lib().bsa_noalloc_scratch_bytes()
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_sparse_attention_fwd_noalloc(q, k, k, idx, cnt, ap, o, lse)
    assert e.value.status == 4 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (o == 0).all()
