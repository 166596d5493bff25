"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before any launch.

Pointers passed here are fake (never dereferenced): every call below returns
from host-side validation, which runs before anything touches the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")
PEAKS_HEADER = os.path.join(ROOT, "include", "bsa_peaks.h")

bsa = pytest.importorskip("dlm_bsa_block_amd")
from dlm_bsa_block_amd import _lib as L  # noqa: E402

FAKE = 0x10000          # 16-byte aligned, never dereferenced


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libbsa.so not built")
    return L.lib()


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
        assert n in L._SIGS, f"binding has no signature for {n}"


def test_peaks_library_exports_every_declared_function():
    from dlm_bsa_block_amd import build as bb
    if not os.path.exists(bb.PEAKS_LIB):
        pytest.skip("libbsa_peaks.so not built")
    plib = ctypes.CDLL(bb.PEAKS_LIB)
    names = _declared_functions(PEAKS_HEADER)
    assert names == ["bsa_peak_hbm_read", "bsa_peak_mfma_bf16", "bsa_peak_mfma_flops"]
    for n in names:
        assert hasattr(plib, n), n
    plib.bsa_peak_mfma_flops.restype = ctypes.c_double
    plib.bsa_peak_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert plib.bsa_peak_mfma_flops(10, 3) == 3 * 4 * 10 * 4 * 32 * 32 * 16 * 2
    # host-side rejection only (nothing reaches the device)
    plib.bsa_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    assert plib.bsa_peak_hbm_read(None, 1 << 20, 64, FAKE, None) == 1
    assert plib.bsa_peak_hbm_read(FAKE, 8, 64, FAKE, None) == 1
    plib.bsa_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert plib.bsa_peak_mfma_bf16(0, 64, FAKE, None) == 1


def test_status_strings(lib):
    assert lib.bsa_status_string(0) == b"ok"
    assert lib.bsa_status_string(3) == b"index-list capacity too small"
    assert lib.bsa_version() >= 1


def _t(B=1, H=8, Lq=64, D=128, dtype=L.BSA_BF16, data=FAKE):
    return L.BsaTensor(data, dtype, B, H, Lq, D, H * Lq * D, Lq * D, D)


def _err(lib):
    return lib.bsa_last_error().decode()


def test_summaries_rejects_bad_arguments(lib):
    x = _t()
    st = lib.bsa_build_block_summaries(ctypes.byref(x), 48, 0, 0, -1, FAKE, None, None)
    assert st == L.BSA_ERR_UNSUPPORTED and "block_size" in _err(lib)
    st = lib.bsa_build_block_summaries(ctypes.byref(_t(D=96)), 64, 0, 0, -1, FAKE, None, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    st = lib.bsa_build_block_summaries(ctypes.byref(_t(data=FAKE + 8)), 64, 0, 0, -1, FAKE, None, None)
    assert st == L.BSA_ERR_INVALID and "aligned" in _err(lib)
    st = lib.bsa_build_block_summaries(ctypes.byref(x), 64, 0, 0, 5, FAKE, None, None)
    assert st == L.BSA_ERR_INVALID            # 64 tokens -> 1 block, 5 requested
    st = lib.bsa_build_block_summaries(ctypes.byref(x), 64, 7, 0, -1, FAKE, None, None)
    assert st == L.BSA_ERR_INVALID
    st = lib.bsa_build_block_summaries(None, 64, 0, 0, -1, FAKE, None, None)
    assert st == L.BSA_ERR_INVALID
    st = lib.bsa_build_block_summaries(ctypes.byref(x), 64, 0, 0, -1, None, None, None)
    assert st == L.BSA_ERR_INVALID
    # empty sequence: nothing to do, nothing launched
    st = lib.bsa_build_block_summaries(ctypes.byref(_t(Lq=0)), 64, 0, 0, -1, FAKE, None, None)
    assert st == L.BSA_OK


def test_select_capacity_and_workspace(lib):
    q = _t(H=32, Lq=1)
    p = bsa.select_params(kv_block=64, q_block=1, topk=13, n_first=1, n_last=2, cap=15)
    st = lib.bsa_select_blocks(ctypes.byref(q), None, FAKE, None, 8, 1024, ctypes.byref(p), None, FAKE, FAKE, None,
                               None, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_CAPACITY and "cap 15 < 16" in _err(lib)
    p.cap = 16
    need = lib.bsa_select_workspace_bytes(ctypes.byref(q), 8, 1024, ctypes.byref(p))
    assert need >= 32 * 1024 * 4
    st = lib.bsa_select_blocks(ctypes.byref(q), None, FAKE, None, 8, 1024, ctypes.byref(p), None, FAKE, FAKE, None,
                               None, FAKE, need - 1, None)
    assert st == L.BSA_ERR_WORKSPACE
    st = lib.bsa_select_blocks(ctypes.byref(q), None, FAKE, None, 7, 1024, ctypes.byref(p), None, FAKE, FAKE, None,
                               None, FAKE, need, None)
    assert st == L.BSA_ERR_INVALID            # 7 does not divide 32
    st = lib.bsa_select_blocks(ctypes.byref(q), None, FAKE, None, 8, 5000, ctypes.byref(p), None, FAKE, FAKE, None,
                               None, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    # dual band needs energies; pooled queries must be f32
    p2 = bsa.select_params(kv_block=128, q_block=128, pooled_q=1, causal=1, topk_num=1, topk_den=10, n_first=1,
                           n_last=1, dual_band=1, cap=256)
    qm = _t(H=32, Lq=256, dtype=L.BSA_F32)
    st = lib.bsa_select_blocks(ctypes.byref(qm), None, FAKE, None, 8, 256, ctypes.byref(p2), None, FAKE, FAKE, None,
                               None, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_INVALID and "energy" in _err(lib)
    st = lib.bsa_select_blocks(ctypes.byref(_t(H=32, Lq=256)), FAKE, FAKE, FAKE, 8, 256, ctypes.byref(p2), None,
                               FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_INVALID and "f32" in _err(lib)
    # union over a 32-row block: capacity bound is min(NB, 32 * 16)
    p3 = bsa.select_params(kv_block=64, q_block=32, topk=16, cap=511)
    st = lib.bsa_select_blocks(ctypes.byref(_t(H=32, Lq=32)), None, FAKE, None, 8, 512, ctypes.byref(p3), None,
                               FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_CAPACITY


def test_attention_rejects_bad_arguments(lib):
    q, k = _t(H=32, Lq=32), _t(H=8, Lq=4096)
    p = bsa.attn_params(kv_block=64, q_block=32, cap=512)
    need = lib.bsa_attention_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(p))
    assert need > 0
    st = lib.bsa_sparse_attention_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                      ctypes.byref(p), None, ctypes.byref(q), FAKE, FAKE, need - 1, None)
    assert st == L.BSA_ERR_WORKSPACE
    qf = _t(H=32, Lq=32, dtype=L.BSA_F32)
    st = lib.bsa_sparse_attention_fwd(ctypes.byref(qf), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                      ctypes.byref(p), None, ctypes.byref(qf), FAKE, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_INVALID            # dtype mismatch q/k
    p96 = bsa.attn_params(kv_block=96, q_block=32, cap=512)
    st = lib.bsa_sparse_attention_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                      ctypes.byref(p96), None, ctypes.byref(q), FAKE, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    # decode path supports G in {1, 2, 4, 8}
    q3, k3 = _t(H=48, Lq=1), _t(H=3, Lq=4096)
    pd = bsa.attn_params(kv_block=64, q_block=1, cap=16)
    st = lib.bsa_sparse_attention_fwd(ctypes.byref(q3), ctypes.byref(k3), ctypes.byref(k3), FAKE, FAKE,
                                      ctypes.byref(pd), None, ctypes.byref(q3), FAKE, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    # o takes q's dtype or f32: an f32 decode query with a bf16 output is refused
    qd, kd, od = _t(H=32, Lq=1, dtype=L.BSA_F32), _t(H=8, Lq=4096, dtype=L.BSA_F32), _t(H=32, Lq=1)
    st = lib.bsa_sparse_attention_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(kd), FAKE, FAKE,
                                      ctypes.byref(pd), None, ctypes.byref(od), FAKE, FAKE, 1 << 30, None)
    assert st == L.BSA_ERR_INVALID and "o must match q" in _err(lib)


def test_attention_noalloc_rejects_on_the_host(lib):
    """The no-workspace attention validates like the workspace form and refuses a call whose
    partials would not fit its static scratch, before touching the device."""
    assert lib.bsa_noalloc_scratch_bytes() == 64 << 20
    q, k = _t(H=32, Lq=4096), _t(H=8, Lq=4096)
    p = bsa.attn_params(kv_block=64, q_block=32, cap=64)
    need = lib.bsa_attention_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(p))
    assert need > lib.bsa_noalloc_scratch_bytes()
    st = lib.bsa_sparse_attention_fwd_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                              ctypes.byref(p), None, ctypes.byref(q), FAKE, None)
    assert st == L.BSA_ERR_WORKSPACE and "static scratch" in _err(lib)
    p96 = bsa.attn_params(kv_block=96, q_block=32, cap=64)
    st = lib.bsa_sparse_attention_fwd_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                              ctypes.byref(p96), None, ctypes.byref(q), FAKE, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    st = lib.bsa_sparse_attention_fwd_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), None, FAKE,
                                              ctypes.byref(p), None, ctypes.byref(q), FAKE, None)
    assert st == L.BSA_ERR_INVALID


def test_threshold_rejects_bad_arguments(lib):
    q, k = _t(H=32, Lq=1024), _t(H=8, Lq=1024)
    for lam, tile, want in ((1.5, 128, L.BSA_ERR_INVALID), (-0.1, 128, L.BSA_ERR_INVALID),
                            (1e-3, 64, L.BSA_ERR_UNSUPPORTED)):
        p = L.BsaThreshParams(0.088, lam, tile, 1)
        st = lib.bsa_threshold_attention_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(p),
                                             ctypes.byref(q), FAKE, None, None, None)
        assert st == want, (lam, tile, _err(lib))
    p = L.BsaThreshParams(0.088, 1e-3, 128, 1)
    kk = _t(H=8, Lq=2048)
    st = lib.bsa_threshold_attention_fwd(ctypes.byref(q), ctypes.byref(kk), ctypes.byref(kk), ctypes.byref(p),
                                         ctypes.byref(q), FAKE, None, None, None)
    assert st == L.BSA_ERR_UNSUPPORTED        # causal needs Lq == L


def test_threshold_decode_rejects_bad_arguments(lib):
    q, k = _t(H=32, Lq=1), _t(H=8, Lq=4096)
    need = lib.bsa_threshold_decode_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 1024)
    assert need > 0

    def call(qq, split, lam, ws=need):
        return lib.bsa_threshold_decode_fwd(ctypes.byref(qq), ctypes.byref(k), ctypes.byref(k), 0.088, lam, split,
                                            ctypes.byref(qq), FAKE, None, None, FAKE, ws, None)
    assert call(q, 1024, 0.3, need - 1) == L.BSA_ERR_WORKSPACE
    assert call(q, 1000, 0.3) == L.BSA_ERR_UNSUPPORTED and "kv_split" in _err(lib)
    assert call(q, 4096, 0.3) == L.BSA_ERR_UNSUPPORTED
    assert call(q, 1024, 1.5) == L.BSA_ERR_INVALID and "lambda" in _err(lib)
    assert call(_t(H=32, Lq=2), 1024, 0.3) == L.BSA_ERR_INVALID and "one query row" in _err(lib)
    assert call(_t(H=24, Lq=1), 1024, 0.3) == L.BSA_ERR_UNSUPPORTED      # group size 3
    # more decision chunks per head than the merge takes (4096 of 4 tiles = 1M keys)
    long_k = _t(H=8, Lq=4096 * 256 + 64)
    big = lib.bsa_threshold_decode_workspace_bytes(ctypes.byref(q), ctypes.byref(long_k), 1024)
    st = lib.bsa_threshold_decode_fwd(ctypes.byref(q), ctypes.byref(long_k), ctypes.byref(long_k), 0.088, 0.3,
                                      1024, ctypes.byref(q), FAKE, None, None, FAKE, big, None)
    assert st == L.BSA_ERR_UNSUPPORTED and "chunks" in _err(lib)


def test_merge_rejects_bad_arguments(lib):
    a, b = _t(H=32, Lq=32, dtype=L.BSA_F32), _t(H=32, Lq=31, dtype=L.BSA_F32)
    st = lib.bsa_merge_attention_states(ctypes.byref(a), FAKE, ctypes.byref(b), FAKE, ctypes.byref(a), FAKE, None)
    assert st == L.BSA_ERR_INVALID and "shape" in _err(lib)
    st = lib.bsa_merge_attention_states(ctypes.byref(a), FAKE, ctypes.byref(a), None, ctypes.byref(a), FAKE, None)
    assert st == L.BSA_ERR_INVALID and "lse" in _err(lib)
    st = lib.bsa_merge_attention_states(ctypes.byref(_t(D=96)), FAKE, ctypes.byref(_t(D=96)), FAKE,
                                        ctypes.byref(_t(D=96)), FAKE, None)
    assert st == L.BSA_ERR_UNSUPPORTED
    st = lib.bsa_merge_attention_states(ctypes.byref(a), FAKE, ctypes.byref(_t(H=32, Lq=32, data=FAKE + 8)), FAKE,
                                        ctypes.byref(a), FAKE, None)
    assert st == L.BSA_ERR_INVALID and "aligned" in _err(lib)
    # no rows: nothing to do, nothing launched
    e = _t(H=32, Lq=0)
    assert lib.bsa_merge_attention_states(ctypes.byref(e), FAKE, ctypes.byref(e), FAKE, ctypes.byref(e), FAKE,
                                          None) == L.BSA_OK


def test_block_attention_merge_rejects_bad_arguments(lib):
    q, kb, o = _t(H=32, Lq=32), _t(H=8, Lq=32), _t(H=32, Lq=32, dtype=L.BSA_F32)

    def call(qq, kk, oo, scale=0.088, lse=FAKE):
        return lib.bsa_block_attention_merge(ctypes.byref(qq), ctypes.byref(kk), ctypes.byref(kk), scale,
                                             ctypes.byref(oo), lse, ctypes.byref(oo), FAKE, None)
    assert call(_t(H=32, Lq=40), _t(H=8, Lq=40), _t(H=32, Lq=40)) == L.BSA_ERR_UNSUPPORTED   # 40 rows
    assert call(q, _t(H=8, Lq=31), o) == L.BSA_ERR_INVALID and "incompatible" in _err(lib)
    assert call(q, _t(H=7, Lq=32), o) == L.BSA_ERR_INVALID                                # 7 does not divide 32
    assert call(q, kb, _t(H=32, Lq=16)) == L.BSA_ERR_INVALID and "shape" in _err(lib)
    assert call(q, kb, o, lse=None) == L.BSA_ERR_INVALID and "lse" in _err(lib)
    assert call(q, kb, o, scale=0.0) == L.BSA_ERR_INVALID and "scale" in _err(lib)
    assert call(_t(H=32, Lq=32, dtype=L.BSA_F32), _t(H=8, Lq=32, dtype=L.BSA_F32), o) == L.BSA_ERR_UNSUPPORTED


def test_window_decode_rejects_bad_arguments(lib):
    q, k = _t(H=32, Lq=1), _t(H=8, Lq=4096)
    p = bsa.attn_params(kv_block=64, q_block=1, cap=16)
    need = lib.bsa_window_decode_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(p), 512)
    assert need > lib.bsa_attention_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(p)) > 0

    def call(qq, pp, window, ws=need):
        return lib.bsa_window_decode_fwd(ctypes.byref(qq), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE,
                                         ctypes.byref(pp), window, None, ctypes.byref(qq), FAKE, FAKE, ws, None)
    assert call(q, p, 512, need - 1) == L.BSA_ERR_WORKSPACE
    assert call(q, p, 0) == L.BSA_ERR_INVALID and "window" in _err(lib)
    p32 = bsa.attn_params(kv_block=64, q_block=32, cap=16)
    assert call(_t(H=32, Lq=32), p32, 512) == L.BSA_ERR_UNSUPPORTED and "decode" in _err(lib)


def test_token_select_and_attention_reject_bad_arguments(lib):
    q, k = _t(H=32, Lq=1), _t(H=8, Lq=4096)
    need = lib.bsa_token_select_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 256)
    assert need >= 32 * 4096 * 4

    def sel(qq, kk, mask=FAKE, layout=0, budget=256, ws=need):
        return lib.bsa_token_select(ctypes.byref(qq), ctypes.byref(kk), mask, layout, budget, FAKE, FAKE, FAKE, ws,
                                    None)
    assert sel(q, k, ws=need - 1) == L.BSA_ERR_WORKSPACE
    assert sel(q, k, mask=None) == L.BSA_ERR_INVALID and "fc_mask" in _err(lib)
    assert sel(q, k, layout=2) == L.BSA_ERR_INVALID
    assert sel(q, k, budget=0) == L.BSA_ERR_INVALID and "budget" in _err(lib)
    assert sel(q, _t(H=8, Lq=65537)) == L.BSA_ERR_UNSUPPORTED
    assert sel(q, k, budget=4096) == L.BSA_ERR_UNSUPPORTED and "budget" in _err(lib)
    assert sel(q, _t(H=8, Lq=65536), budget=2048) == L.BSA_ERR_UNSUPPORTED         # 16 parts x 2048 > 16384
    assert sel(_t(H=32, Lq=2), k) == L.BSA_ERR_INVALID and "one query row" in _err(lib)
    assert sel(_t(H=32, Lq=1, D=64), _t(H=8, Lq=4096, D=64)) == L.BSA_ERR_UNSUPPORTED
    wa = lib.bsa_token_attention_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 256)
    assert wa > 0

    def att(cap=256, scale=0.088, ws=wa, o=q):
        return lib.bsa_token_attention_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), FAKE, FAKE, cap, scale,
                                           ctypes.byref(o), FAKE, FAKE, ws, None)
    assert att(ws=wa - 1) == L.BSA_ERR_WORKSPACE
    assert att(cap=0) == L.BSA_ERR_INVALID
    assert att(scale=float("inf")) == L.BSA_ERR_INVALID
    assert att(o=_t(H=32, Lq=2)) == L.BSA_ERR_INVALID and "o must match" in _err(lib)


def test_select_refresh_rejects_bad_arguments(lib):
    q, k = _t(H=32, Lq=1), _t(H=8, Lq=4096)
    p = bsa.select_params(kv_block=64, q_block=1, topk=13, n_first=1, n_last=2, cap=16, q_pos0=4095)

    def call(kk, blk, pp=p, nb=64):
        return lib.bsa_select_blocks_refresh(ctypes.byref(kk), blk, ctypes.byref(q), FAKE, None, 8, nb,
                                             ctypes.byref(pp), None, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert call(k, 64) == L.BSA_ERR_INVALID and "refresh_block" in _err(lib)
    assert call(k, -1) == L.BSA_ERR_INVALID
    assert call(_t(H=8, Lq=4000), 62, nb=64) == L.BSA_ERR_INVALID and "num_kv_blocks" in _err(lib)
    assert call(_t(H=4, Lq=4096), 63) == L.BSA_ERR_INVALID
    pd = bsa.select_params(kv_block=64, q_block=1, topk=13, dual_band=1, cap=16)
    assert call(k, 63, pp=pd) == L.BSA_ERR_UNSUPPORTED
    pc = bsa.select_params(kv_block=64, q_block=1, topk=13, causal=1, q_pos0=100, cap=16)
    assert call(k, 63, pp=pc) == L.BSA_ERR_INVALID and "visible" in _err(lib)


def test_active_rows_rejects_mismatch(lib):
    a, b = _t(H=32, Lq=32), _t(H=32, Lq=31)
    st = lib.bsa_active_rows(ctypes.byref(a), ctypes.byref(b), 0.1, FAKE, None, None)
    assert st == L.BSA_ERR_INVALID
    st = lib.bsa_active_rows(ctypes.byref(a), ctypes.byref(a), float("nan"), FAKE, None, None)
    assert st == L.BSA_ERR_INVALID


def test_product_path_does_not_import_oracle():
    """The library binding never reaches the CPU oracle."""
    import sys
    pkg = os.path.join(ROOT, "dlm_bsa_block_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "oracle" not in src.replace("oracle/", ""), f
    assert "oracle" not in sys.modules.get("dlm_bsa_block_amd").__dict__


def test_attention_workspace_layout(lib):
    """The attention workspaces start with a fixed 64 KiB counter region whenever
    they hold split partials, so calls of any shape find the counters where the
    previous call left them; the direct prefill path needs no workspace."""
    COUNTERS = 65536
    pd = bsa.attn_params(kv_block=64, q_block=1, cap=16)
    k = _t(H=8, Lq=65536)
    # decode of bf16 rows with D = 128 (the matrix-core form): 16 slices of 64 tokens per (row, group),
    # partials of 8 rows x 16 slices x 4 heads
    one = lib.bsa_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=1)), ctypes.byref(k), ctypes.byref(pd))
    parts = 8 * 16 * 4
    assert one == COUNTERS + ((parts * 128 * 4 + 255) // 256) * 256 + ((parts * 2 * 4 + 255) // 256) * 256
    # more rows than counters (8 x 129 > 1024): the region is still there, the combine merges instead;
    # with 1032 lists in one launch each list is one slice of all its 1024 tokens (a launch with
    # many lists keeps about 512 workgroups), so the partials hold one slice per (row, group)
    many = lib.bsa_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=129)), ctypes.byref(k), ctypes.byref(pd))
    parts = 8 * 129 * 1 * 4
    assert many == COUNTERS + ((parts * 128 * 4 + 255) // 256) * 256 + ((parts * 2 * 4 + 255) // 256) * 256
    # 32 rows (256 lists): slices of 512 tokens, 2 per list
    mid = lib.bsa_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=32)), ctypes.byref(k), ctypes.byref(pd))
    parts = 8 * 32 * 2 * 4
    assert mid == COUNTERS + ((parts * 128 * 4 + 255) // 256) * 256 + ((parts * 2 * 4 + 255) // 256) * 256
    # MFMA split of a 32-row block: counters too (one workspace may serve both kinds of call)
    ps = bsa.attn_params(kv_block=64, q_block=32, cap=512)
    split = lib.bsa_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=32)), ctypes.byref(k), ctypes.byref(ps))
    assert split > COUNTERS
    # direct prefill (128-row blocks): no partials, no workspace
    pp = bsa.attn_params(kv_block=128, q_block=128, cap=64)
    assert lib.bsa_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=4096)), ctypes.byref(_t(H=8, Lq=4096)),
                                             ctypes.byref(pp)) == 0
    # the window decode and the token attention lay theirs out the same way
    win = lib.bsa_window_decode_workspace_bytes(ctypes.byref(_t(H=32, Lq=1)), ctypes.byref(k), ctypes.byref(pd), 512)
    assert win > one                                  # the window adds its slices after the list's
    tok = lib.bsa_token_attention_workspace_bytes(ctypes.byref(_t(H=32, Lq=1)), ctypes.byref(k), 256)
    parts_t = 32 * 8                                  # 32 query heads x 8 slices of 32 tokens
    assert tok == COUNTERS + ((parts_t * 128 * 4 + 255) // 256) * 256 + ((parts_t * 2 * 4 + 255) // 256) * 256
