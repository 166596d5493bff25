"""Query-aware block-sparse attention on MI355X: thin torch binding of libbsa.

Each function has the name of the C entry point it wraps and only marshals
arguments: tensors become (device pointer, shape, strides) descriptors, the
current torch stream becomes the HIP stream, and outputs/workspaces are
allocated with torch.  Every step of the computation runs in the HIP kernels
of libbsa.so; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (  # noqa: F401
    BSA_BF16, BSA_F32, BSA_ROPE_HALF, BSA_ROPE_INTERLEAVED, BsaAttnParams, BsaError, BsaSelectParams,
    BsaTensor, BsaThreshParams, check, lib,
)

__all__ = ["bsa_build_block_summaries", "bsa_select_blocks", "bsa_active_rows", "bsa_merge_attention_states",
           "bsa_block_attention_merge", "bsa_window_decode_fwd", "bsa_window_decode_workspace_bytes",
           "bsa_token_select", "bsa_token_attention_fwd", "bsa_select_blocks_refresh",
           "bsa_sparse_attention_fwd", "bsa_sparse_attention_fwd_noalloc", "bsa_decode_step",
           "bsa_decode_step_workspace_bytes",
           "bsa_threshold_attention_fwd", "bsa_threshold_decode_fwd", "bsa_select_workspace_bytes",
           "bsa_attention_workspace_bytes", "bsa_threshold_decode_workspace_bytes",
           "BsaError", "tensor_desc", "select_params", "attn_params", "lib"]

_DT = {torch.bfloat16: BSA_BF16, torch.float32: BSA_F32}


def tensor_desc(t: torch.Tensor) -> BsaTensor:
    """Descriptor of a 4-D [B, H, L, D] device tensor with a contiguous last dim."""
    if t.dim() != 4:
        raise ValueError(f"expected a 4-D [B, H, L, D] tensor, got shape {tuple(t.shape)}")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the last dim must be contiguous")
    B, H, L, D = t.shape
    return BsaTensor(t.data_ptr(), _DT[t.dtype], B, H, L, D, t.stride(0), t.stride(1), t.stride(2))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def select_params(kv_block, q_block=1, q_pos0=0, q_len=0, causal=0, pooled_q=0, topk=0, topk_num=0, topk_den=1,
                  n_first=0, n_last=0, dual_band=0, layout=BSA_ROPE_HALF, scale=None, cap=None, D=128):
    return BsaSelectParams(kv_block, q_block, q_pos0, q_len, causal, pooled_q, topk, topk_num, topk_den, n_first,
                           n_last, dual_band, layout, 1.0 / math.sqrt(D) if scale is None else scale,
                           0 if cap is None else cap)


def attn_params(kv_block, q_block, cap, q_pos0=0, causal=0, scale=None, D=128):
    return BsaAttnParams(1.0 / math.sqrt(D) if scale is None else scale, kv_block, q_block, q_pos0, causal, cap)


def list_capacity(NB, rows_per_block, p: BsaSelectParams) -> int:
    """Smallest capacity the selection accepts: min(NB, rows * (k' + forced))."""
    kp = -(-(p.topk_num * NB) // p.topk_den) if p.topk_num > 0 else p.topk
    return min(NB, rows_per_block * (kp + p.n_first + p.n_last))


# --------------------------------------------------------------- summaries ---
def bsa_build_block_summaries(x: torch.Tensor, block_size: int, layout: int = BSA_ROPE_HALF, first_block: int = 0,
                              num_blocks: int = -1, mean: torch.Tensor | None = None,
                              energy: torch.Tensor | None = None, with_energy: bool = True):
    B, H, L, D = x.shape
    NB = -(-L // block_size)
    if mean is None:
        mean = torch.empty((B, H, NB, D), dtype=torch.float32, device=x.device)
    if energy is None and with_energy:
        energy = torch.empty((B, H, NB, 2), dtype=torch.float32, device=x.device)
    xd = tensor_desc(x)
    check(lib().bsa_build_block_summaries(ctypes.byref(xd), block_size, layout, first_block, num_blocks,
                                          mean.data_ptr(), _ptr(energy), _stream()), "bsa_build_block_summaries")
    return mean, energy


# --------------------------------------------------------------- selection ---
def bsa_select_workspace_bytes(q: torch.Tensor, num_kv_heads: int, num_kv_blocks: int, p: BsaSelectParams) -> int:
    qd = tensor_desc(q)
    return lib().bsa_select_workspace_bytes(ctypes.byref(qd), num_kv_heads, num_kv_blocks, ctypes.byref(p))


def bsa_select_blocks(q: torch.Tensor, k_mean: torch.Tensor, p: BsaSelectParams, k_energy=None, q_energy=None,
                      row_mask=None, want_row_picks=False, want_tau=False, workspace=None, idx=None, cnt=None):
    """Returns (idx [B,Hkv,NQB,cap] int32, cnt [B,Hkv,NQB] int32, row_picks or None, tau or None).

    idx, cnt and workspace may be passed in (e.g. for graph capture, where
    nothing may be allocated)."""
    B, Hkv, NB, D = k_mean.shape
    Hq = q.shape[1]
    if p.pooled_q:
        NQB = q.shape[2]
        R = NQB
    else:
        Lq = q.shape[2]
        NQB = -(-Lq // p.q_block)
        R = Lq
    if p.cap <= 0:
        p.cap = list_capacity(NB, 1 if p.pooled_q else min(p.q_block, q.shape[2]), p)
    dev = q.device
    if idx is None:
        idx = torch.empty((B, Hkv, NQB, p.cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv, NQB), dtype=torch.int32, device=dev)
    rp = torch.empty((B, Hkv, R, p.cap), dtype=torch.int32, device=dev) if want_row_picks else None
    tau = torch.empty((B, Hq, 2), dtype=torch.float32, device=dev) if want_tau else None
    qd = tensor_desc(q)
    need = lib().bsa_select_workspace_bytes(ctypes.byref(qd), Hkv, NB, ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)   # no initial contents needed
    check(lib().bsa_select_blocks(ctypes.byref(qd), _ptr(q_energy), k_mean.data_ptr(), _ptr(k_energy), Hkv, NB,
                                  ctypes.byref(p), _ptr(row_mask), idx.data_ptr(), cnt.data_ptr(), _ptr(rp),
                                  _ptr(tau), workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_select_blocks")
    return idx, cnt, rp, tau


# ------------------------------------------------------------- active rows ---
def bsa_active_rows(q_cur: torch.Tensor, q_prev: torch.Tensor, theta: float, want_mse=True, mask=None, mse=None):
    B, H, R, D = q_cur.shape
    if mask is None:
        mask = torch.empty((B, R), dtype=torch.uint8, device=q_cur.device)
    if mse is None and want_mse:
        mse = torch.empty((B, R), dtype=torch.float32, device=q_cur.device)
    a, b = tensor_desc(q_cur), tensor_desc(q_prev)
    check(lib().bsa_active_rows(ctypes.byref(a), ctypes.byref(b), theta, mask.data_ptr(), _ptr(mse), _stream()),
          "bsa_active_rows")
    return mask, mse


def bsa_merge_attention_states(o_a, lse_a, o_b, lse_b, o=None, lse=None):
    """Returns (o, lse): the state over the union of two disjoint key sets.
    o may be o_a or o_b and lse may be lse_a or lse_b (in place)."""
    if o is None:
        o = torch.empty_like(o_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    a, b, c = tensor_desc(o_a), tensor_desc(o_b), tensor_desc(o)
    check(lib().bsa_merge_attention_states(ctypes.byref(a), lse_a.data_ptr(), ctypes.byref(b), lse_b.data_ptr(),
                                           ctypes.byref(c), lse.data_ptr(), _stream()), "bsa_merge_attention_states")
    return o, lse


def bsa_block_attention_merge(q, kb, vb, o_pre, lse_pre, scale=None, o=None, lse=None):
    """Returns (o, lse): attention of the block's rows over the block's own keys
    merged with the cached prefix state (o may be o_pre, lse may be lse_pre)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[3])
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty_like(lse_pre)
    qd, kd, vd, pd, od = tensor_desc(q), tensor_desc(kb), tensor_desc(vb), tensor_desc(o_pre), tensor_desc(o)
    check(lib().bsa_block_attention_merge(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), scale,
                                          ctypes.byref(pd), lse_pre.data_ptr(), ctypes.byref(od), lse.data_ptr(),
                                          _stream()), "bsa_block_attention_merge")
    return o, lse


# --------------------------------------------------------------- attention ---
def bsa_attention_workspace_bytes(q: torch.Tensor, k: torch.Tensor, p: BsaAttnParams) -> int:
    qd, kd = tensor_desc(q), tensor_desc(k)
    return lib().bsa_attention_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(p))


def bsa_sparse_attention_fwd(q, k, v, idx, cnt, p: BsaAttnParams, row_mask=None, o=None, lse=None, workspace=None):
    """Returns (o, lse).  Rows with row_mask = 0 keep whatever o/lse held."""
    B, Hq, Lq, D = q.shape
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((B, Hq, Lq), dtype=torch.float32, device=q.device)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    need = lib().bsa_attention_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        # the arrival counters at its front must be zero on the first call (calls leave them zero)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    check(lib().bsa_sparse_attention_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), idx.data_ptr(),
                                         cnt.data_ptr(), ctypes.byref(p), _ptr(row_mask), ctypes.byref(od),
                                         lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_sparse_attention_fwd")
    return o, lse


def bsa_sparse_attention_fwd_noalloc(q, k, v, idx, cnt, p: BsaAttnParams, o, lse, row_mask=None):
    """bsa_sparse_attention_fwd with its partials in the library's static device scratch: nothing is
    allocated, so o and lse must be given.  Returns (o, lse)."""
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    check(lib().bsa_sparse_attention_fwd_noalloc(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                                                 idx.data_ptr(), cnt.data_ptr(), ctypes.byref(p), _ptr(row_mask),
                                                 ctypes.byref(od), lse.data_ptr(), _stream()),
          "bsa_sparse_attention_fwd_noalloc")
    return o, lse


def bsa_select_blocks_refresh(k, refresh_block: int, q, k_mean, p: BsaSelectParams, k_energy=None, row_mask=None,
                              want_row_picks=False, workspace=None, idx=None, cnt=None):
    """bsa_build_block_summaries of block `refresh_block` (into k_mean / k_energy) and bsa_select_blocks, in
    the selection's launches.  Returns (idx, cnt, row_picks or None)."""
    B, Hkv, NB, D = k_mean.shape
    Lq = q.shape[2]
    NQB = -(-Lq // p.q_block)
    if p.cap <= 0:
        p.cap = list_capacity(NB, min(p.q_block, Lq), p)
    dev = q.device
    if idx is None:
        idx = torch.empty((B, Hkv, NQB, p.cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv, NQB), dtype=torch.int32, device=dev)
    rp = torch.empty((B, Hkv, Lq, p.cap), dtype=torch.int32, device=dev) if want_row_picks else None
    qd, kd = tensor_desc(q), tensor_desc(k)
    need = lib().bsa_select_workspace_bytes(ctypes.byref(qd), Hkv, NB, ctypes.byref(p))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)   # no initial contents needed
    check(lib().bsa_select_blocks_refresh(ctypes.byref(kd), refresh_block, ctypes.byref(qd), k_mean.data_ptr(),
                                          _ptr(k_energy), Hkv, NB, ctypes.byref(p), _ptr(row_mask), idx.data_ptr(),
                                          cnt.data_ptr(), _ptr(rp), workspace.data_ptr(), workspace.numel(),
                                          _stream()), "bsa_select_blocks_refresh")
    return idx, cnt, rp


def bsa_decode_step_workspace_bytes(q, k, p: BsaSelectParams) -> int:
    return int(lib().bsa_decode_step_workspace_bytes(ctypes.byref(tensor_desc(q)), ctypes.byref(tensor_desc(k)),
                                                     ctypes.byref(p)))


def bsa_decode_step(q, k, v, k_mean, p: BsaSelectParams, refresh_block: int = -1, k_energy=None, idx=None, cnt=None,
                    o=None, lse=None, workspace=None):
    """Selection (with the summary of block ``refresh_block`` pooled first, unless -1) and attention over the
    selected blocks for decode rows.  Returns (idx [B,Hkv,Lq,cap], cnt [B,Hkv,Lq], o, lse [B,Hq,Lq])."""
    B, Hq, Lq, D = q.shape
    Hkv, NB = k_mean.shape[1], k_mean.shape[2]
    if p.cap <= 0:
        p.cap = list_capacity(NB, 1, p)
    dev = q.device
    if idx is None:
        idx = torch.empty((B, Hkv, Lq, p.cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv, Lq), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
    need = bsa_decode_step_workspace_bytes(q, k, p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)   # no initial contents needed
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    check(lib().bsa_decode_step(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), k_mean.data_ptr(),
                                _ptr(k_energy), refresh_block, ctypes.byref(p), idx.data_ptr(), cnt.data_ptr(),
                                ctypes.byref(od), lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream()), "bsa_decode_step")
    return idx, cnt, o, lse


def bsa_denoise_step_workspace_bytes(q, k, p: BsaSelectParams) -> int:
    return int(lib().bsa_denoise_step_workspace_bytes(ctypes.byref(tensor_desc(q)), ctypes.byref(tensor_desc(k)),
                                                      ctypes.byref(p)))


def bsa_denoise_step(q, q_prev, theta: float, k_mean, k, v, kb, vb, p: BsaSelectParams, cache_o, cache_lse,
                     row_mask=None, mse=None, want_mse=False, idx=None, cnt=None, o=None, lse=None, workspace=None):
    """One locality-pruned denoising step: active rows, their block selection, prefix attention of the active
    rows into (cache_o, cache_lse) and the block attention merged with the prefix state for every row.
    Returns (row_mask [B,R], mse or None, idx [B,Hkv,1,cap], cnt [B,Hkv,1], o, lse [B,Hq,R])."""
    B, Hq, R, D = q.shape
    Hkv, NB = k_mean.shape[1], k_mean.shape[2]
    if p.cap <= 0:
        p.cap = list_capacity(NB, R, p)
    dev = q.device
    if row_mask is None:
        row_mask = torch.empty((B, R), dtype=torch.uint8, device=dev)
    if mse is None and want_mse:
        mse = torch.empty((B, R), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, Hkv, 1, p.cap), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((B, Hkv, 1), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, R), dtype=torch.float32, device=dev)
    need = bsa_denoise_step_workspace_bytes(q, k, p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)   # no initial contents needed
    qd, pd, kd, vd = tensor_desc(q), tensor_desc(q_prev), tensor_desc(k), tensor_desc(v)
    kbd, vbd, cd, od = tensor_desc(kb), tensor_desc(vb), tensor_desc(cache_o), tensor_desc(o)
    check(lib().bsa_denoise_step(ctypes.byref(qd), ctypes.byref(pd), theta, k_mean.data_ptr(), ctypes.byref(kd),
                                 ctypes.byref(vd), ctypes.byref(kbd), ctypes.byref(vbd), ctypes.byref(p),
                                 ctypes.byref(cd), cache_lse.data_ptr(), row_mask.data_ptr(), _ptr(mse),
                                 idx.data_ptr(), cnt.data_ptr(), ctypes.byref(od), lse.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream()), "bsa_denoise_step")
    return row_mask, mse, idx, cnt, o, lse


def bsa_window_decode_workspace_bytes(q, k, p: BsaAttnParams, window: int) -> int:
    qd, kd = tensor_desc(q), tensor_desc(k)
    return lib().bsa_window_decode_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(p), window)


def bsa_window_decode_fwd(q, k, v, idx, cnt, p: BsaAttnParams, window: int, gates=None, o=None, lse=None,
                          workspace=None):
    """Returns (o, lse [B,Hq,Lq,2]): selected blocks and the sliding window, o = g_sel O_sel + g_win O_win."""
    B, Hq, Lq, D = q.shape
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((B, Hq, Lq, 2), dtype=torch.float32, device=q.device)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    need = bsa_window_decode_workspace_bytes(q, k, p, window)
    if workspace is None or workspace.numel() < need:
        # the arrival counters at its front must be zero on the first call (calls leave them zero)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    check(lib().bsa_window_decode_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), idx.data_ptr(),
                                      cnt.data_ptr(), ctypes.byref(p), window, _ptr(gates), ctypes.byref(od),
                                      lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_window_decode_fwd")
    return o, lse


def bsa_token_select_workspace_bytes(q, k, budget: int) -> int:
    qd, kd = tensor_desc(q), tensor_desc(k)
    return lib().bsa_token_select_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), budget)


def bsa_token_attention_workspace_bytes(q, k, cap: int) -> int:
    qd, kd = tensor_desc(q), tensor_desc(k)
    return lib().bsa_token_attention_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), cap)


def bsa_token_select(q, k, fc_mask, budget: int, layout: int = BSA_ROPE_HALF, idx=None, cnt=None, workspace=None):
    """Returns (idx [B,Hq,budget] int32 ascending, cnt [B,Hq] int32): each head's best tokens by q . k over
    the frequency chunks marked in fc_mask [Hq, D/2] (uint8, on the device)."""
    B, Hq = q.shape[:2]
    if idx is None:
        idx = torch.empty((B, Hq, budget), dtype=torch.int32, device=q.device)
    if cnt is None:
        cnt = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    qd, kd = tensor_desc(q), tensor_desc(k)
    need = bsa_token_select_workspace_bytes(q, k, budget)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    check(lib().bsa_token_select(ctypes.byref(qd), ctypes.byref(kd), fc_mask.data_ptr(), layout, budget,
                                 idx.data_ptr(), cnt.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_token_select")
    return idx, cnt


def bsa_token_attention_fwd(q, k, v, idx, cnt, scale=None, o=None, lse=None, workspace=None):
    """Returns (o, lse): each query head over its own tokens (idx [B,Hq,Lq,cap] or [B,Hq,cap] for Lq = 1)."""
    B, Hq, Lq, D = q.shape
    cap = idx.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((B, Hq, Lq), dtype=torch.float32, device=q.device)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    need = bsa_token_attention_workspace_bytes(q, k, cap)
    if workspace is None or workspace.numel() < need:
        # the arrival counters at its front must be zero on the first call (calls leave them zero)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    check(lib().bsa_token_attention_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), idx.data_ptr(),
                                        cnt.data_ptr(), cap, scale, ctypes.byref(od), lse.data_ptr(),
                                        workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_token_attention_fwd")
    return o, lse


def bsa_threshold_attention_fwd(q, k, v, lam: float, scale: float | None = None, tile: int = 128, causal: int = 1,
                                want_keep_map=False, o=None, lse=None, kept=None):
    """Returns (o, lse, kept_tiles [B,Hq,NQT] int32, keep_map [B,Hq,NQT,NKT] uint8 or None)."""
    B, Hq, Lq, D = q.shape
    L = k.shape[2]
    NQT, NKT = -(-Lq // tile), -(-L // tile)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if kept is None:
        kept = torch.empty((B, Hq, NQT), dtype=torch.int32, device=q.device)
    km = torch.zeros((B, Hq, NQT, NKT), dtype=torch.uint8, device=q.device) if want_keep_map else None
    p = BsaThreshParams(1.0 / math.sqrt(D) if scale is None else scale, lam, tile, causal)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    check(lib().bsa_threshold_attention_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(p),
                                            ctypes.byref(od), lse.data_ptr(), kept.data_ptr(), _ptr(km), _stream()),
          "bsa_threshold_attention_fwd")
    return o, lse, kept, km


# -------------------------------------------------------- threshold decode ---
def bsa_threshold_decode_workspace_bytes(q: torch.Tensor, k: torch.Tensor, kv_split: int) -> int:
    return int(lib().bsa_threshold_decode_workspace_bytes(ctypes.byref(tensor_desc(q)), ctypes.byref(tensor_desc(k)),
                                                          kv_split))


def bsa_threshold_decode_fwd(q, k, v, lam: float, scale: float | None = None, kv_split: int = 1024,
                             want_keep_map=False, o=None, lse=None, kept=None, workspace=None):
    """One query row per head over all keys.  Returns (o, lse [B,Hq,1], kept_tiles [B,Hq] int32,
    keep_map [B,Hq,ceil(L/64)] uint8 or None)."""
    B, Hq, Lq, D = q.shape
    L = k.shape[2]
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if kept is None:
        kept = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    km = torch.zeros((B, Hq, -(-L // 64)), dtype=torch.uint8, device=q.device) if want_keep_map else None
    need = bsa_threshold_decode_workspace_bytes(q, k, kv_split)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    qd, kd, vd, od = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(o)
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    check(lib().bsa_threshold_decode_fwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), sc, lam, kv_split,
                                         ctypes.byref(od), lse.data_ptr(), kept.data_ptr(), _ptr(km),
                                         workspace.data_ptr(), workspace.numel(), _stream()),
          "bsa_threshold_decode_fwd")
    return o, lse, kept, km
