// Gather-by-block-index attention with bf16 MFMA tiles (FASA page sec. 2:
// full head-dim attention over only the selected tokens, at their original
// positions).  Used for
//   * causal sparse prefill: one workgroup per (query block of 128 rows, query
//     head) walking the group's list of KV tiles; workgroups that share a KV
//     group are placed on the same XCD, heads of one query block next to each
//     other, so their K/V tiles are re-read from that XCD's L2;
//   * the denoising step: one workgroup per (slice of the list, query block,
//     KV group) holding the block's active (row, head) pairs as up to 128
//     query vectors, writing split partials for the combine (LoSA sec. 2:
//     only active rows recompute, over the block's union).
// K/V tiles are staged in LDS (V transposed) and shared by the 4 waves; each
// wave owns 32 query vectors.  Online softmax in fp32 with exp2; the running
// max and sum are lane-local (see mfma_tile.cuh).
#include <algorithm>

#include "internal.h"
#include "mfma_tile.cuh"
#include "split.h"

namespace bsa {

struct GatherArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl;
  const int32_t* idx;
  const int32_t* cnt;
  int B, cap, NQB, Hkv, G, L, Lq, q_block, q_pos0, causal;
  float c2;                       // scale * log2(e)
  const uint8_t* row_mask;
  uint16_t* o;
  int64_t osb, osh, osl;
  float* lse;
  float* part_o;
  float* part_ml;
  int items;
};

template <int KVB, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gather_mfma_kernel(GatherArgs a) {
  constexpr int VST = VtStride<KVB>::value;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KVB * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * VST];
  __shared__ int qv_row[128], qv_head[128], qv_full[128];
  __shared__ int n_qv_sh;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31;
  int b, g, qb, item = 0, hl_fixed = 0;
  if (SPLIT) {
    item = blockIdx.x;
    qb = blockIdx.y;
    b = blockIdx.z / a.Hkv;
    g = blockIdx.z - b * a.Hkv;
  } else {
    // XCD-aware order: workgroup n runs on XCD n % 8; give each XCD a contiguous
    // run of (batch, group, query block descending, head) work items.
    const int total = gridDim.x;
    const int n = blockIdx.x;
    const int i = (total % 8 == 0) ? (n % 8) * (total / 8) + n / 8 : n;
    hl_fixed = i % a.G;
    const int rest = i / a.G;
    qb = a.NQB - 1 - rest % a.NQB;
    const int bgi = rest / a.NQB;
    b = bgi / a.Hkv;
    g = bgi - b * a.Hkv;
  }
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  const int n_list = a.cnt[li];
  int e0 = 0, e1 = n_list;
  if (SPLIT) {
    e0 = item * kSplitBlocks;
    if (e0 >= n_list) return;
    e1 = min(n_list, e0 + kSplitBlocks);
  }

  // query vectors of this workgroup
  if (SPLIT) {
    if (w == 0) {
      const int row = qb * a.q_block + lane;
      const bool act = lane < a.q_block && row < a.Lq && (!a.row_mask || a.row_mask[(int64_t)b * a.Lq + row]);
      const unsigned long long m = __ballot(act);
      if (act) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        for (int hh = 0; hh < a.G; ++hh) {
          qv_row[rank * a.G + hh] = row;
          qv_head[rank * a.G + hh] = hh;
          qv_full[rank * a.G + hh] = lane * a.G + hh;
        }
      }
      if (lane == 0) n_qv_sh = __popcll(m) * a.G;
    }
    __syncthreads();
  }
  const int n_qv = SPLIT ? n_qv_sh : 0;
  const int qv = 32 * w + r32;
  bool valid;
  int row, h;
  if (SPLIT) {
    valid = qv < n_qv;
    row = valid ? qv_row[qv] : 0;
    h = g * a.G + (valid ? qv_head[qv] : 0);
  } else {
    const int rl = qv;
    row = qb * a.q_block + rl;
    valid = rl < a.q_block && row < a.Lq;
    h = g * a.G + hl_fixed;
  }
  const bool wave_busy = SPLIT ? (32 * w < n_qv) : (32 * w < a.q_block && qb * a.q_block + 32 * w < a.Lq);
  const int qpos = a.q_pos0 + row;
  // smallest query position of the wave (for deciding whether a tile needs the causal mask)
  int wave_min_pos = valid ? qpos : 0x7FFFFFFF;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_min_pos = min(wave_min_pos, wave_xor(wave_min_pos, m));

  bf16x8 qf[8];
  load_q_frag(a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)row * a.qsl, valid, qf);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  for (int e = e0; e < e1; ++e) {
    const int j = a.idx[li * a.cap + e];
    const int key0 = j * KVB;
    const int nk = (j < 0 || key0 >= a.L) ? 0 : min(KVB, a.L - key0);   // a bad index reads nothing
    stage_kv_tile<KVB>(kbg + (int64_t)key0 * a.ksl, a.ksl, vbg + (int64_t)key0 * a.vsl, a.vsl, nk, Ks, Vt, true, true);
    __syncthreads();
    if (wave_busy) {
      f32x16 s[KVB / 32];
      qk_tile<KVB>(Ks, qf, s);
      const bool need_mask = nk < KVB || (a.causal && key0 + KVB - 1 > wave_min_pos);
      if (need_mask) {
        // largest visible key offset of this lane's query in the tile
        int lim = nk - 1;
        if (a.causal) lim = min(lim, qpos - key0);
        mask_tile<KVB / 32>(s, lim);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KVB / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      mx = fmaxf(mx, wave_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.c2);
      const float msafe = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - msafe);
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < KVB / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pr = fast_exp2(fmaf(s[kt][i], a.c2, -msafe));
          s[kt][i] = pr;
          ls += pr;
        }
      l_run = fmaf(l_run, alpha, ls);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      pv_tile<KVB>(Vt, s, o);
    }
    __syncthreads();
  }

  if (!wave_busy) return;
  const float l_tot = l_run + wave_xor(l_run, 32);
  if (!SPLIT) {
    if (!valid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = a.o + (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)row * a.osl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = o_dim(dt, 4 * i4);
        u32x2 pk = {pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv),
                    pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
    if (lane < 32)
      a.lse[((int64_t)b * a.Hkv * a.G + h) * a.Lq + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    if (!valid) return;
    const int QV = a.q_block * a.G;
    const int64_t pi = (li * a.items + item) * QV + qv_full[qv];
    float* po = a.part_o + pi * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = o_dim(dt, 4 * i4);
        f32x4 v4 = {o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(po + d) = v4;
      }
    if (lane < 32) {
      a.part_ml[pi * 2] = m_run;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

void launch_gather(const GatherArgs& a, int kv_block, bool split, hipStream_t s) {
  if (split) {
    dim3 grid(a.items, a.NQB, a.B * a.Hkv);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, true>), grid, dim3(256), 0, s, a);
  } else {
    dim3 grid(a.B * a.Hkv * a.NQB * a.G);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<128, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, false>), grid, dim3(256), 0, s, a);
  }
}

// ------------------------------------------------------------------- host ---
bool plan_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_attn_params& p, AttnPlan& pl) {
  pl.B = q.B;
  pl.Hq = q.H;
  pl.Hkv = k.H;
  pl.G = q.H / k.H;
  pl.D = q.D;
  pl.Lq = q.L;
  pl.L = k.L;
  pl.NQB = (int)ceil_div(q.L, p.q_block);
  if (p.q_block == 1) {
    pl.kind = 0;
    const int64_t toks = (int64_t)p.cap * p.kv_block;
    // slices of at least kDecMinSlice tokens (whole chunks), at most kDecMaxItems of them
    const int64_t per = std::max<int64_t>(kDecMinSlice / kDecTok, ceil_div(ceil_div(toks, kDecTok), kDecMaxItems));
    pl.tok_per_item = (int)(per * kDecTok);
    pl.items = (int)ceil_div(toks, pl.tok_per_item);
    pl.qv = pl.G;
  } else if (p.q_block * pl.G <= 128 && p.q_block <= 64) {
    pl.kind = 2;
    pl.items = (int)ceil_div(p.cap, kSplitBlocks);
    pl.qv = p.q_block * pl.G;
  } else {
    pl.kind = 1;
    pl.items = 0;
    pl.qv = 0;
  }
  pl.part_bytes = 0;
  if (pl.kind != 1) {
    const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
    pl.part_bytes = align256(n * pl.D * 4) + align256(n * 2 * 4);
  }
  return true;
}

void launch_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                      const int32_t* cnt, const bsa_attn_params& p, const AttnPlan& pl, const uint8_t* row_mask,
                      const bsa_tensor& o, float* lse, void* ws, hipStream_t s) {
  const float c2 = p.scale * kLog2e;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = nullptr;
  if (pl.kind != 1) {
    const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
    part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(n * pl.D * 4));
  }
  if (pl.kind == 0) {
    DecArgs a;
    a.q = static_cast<const uint8_t*>(q.data);
    a.k = static_cast<const uint8_t*>(k.data);
    a.v = static_cast<const uint8_t*>(v.data);
    a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
    a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
    a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
    a.idx = idx; a.cnt = cnt; a.cap = p.cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.L = pl.L;
    a.kv_block = p.kv_block; a.causal = p.causal; a.q_pos0 = p.q_pos0; a.Lq = pl.Lq; a.items = pl.items;
    a.tok_per_item = pl.tok_per_item;
    a.c2 = c2; a.row_mask = row_mask; a.part_o = part_o; a.part_ml = part_ml;
    launch_decode(a, q.dtype, pl.D, pl.G, pl.B, s);
  } else {
    GatherArgs a;
    a.q = static_cast<const uint16_t*>(q.data);
    a.k = static_cast<const uint16_t*>(k.data);
    a.v = static_cast<const uint16_t*>(v.data);
    a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
    a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
    a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
    a.idx = idx; a.cnt = cnt; a.B = pl.B; a.cap = p.cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.G = pl.G;
    a.L = pl.L; a.Lq = pl.Lq; a.q_block = p.q_block; a.q_pos0 = p.q_pos0; a.causal = p.causal; a.c2 = c2;
    a.row_mask = row_mask;
    a.o = static_cast<uint16_t*>(o.data); a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
    a.lse = lse; a.part_o = part_o; a.part_ml = part_ml; a.items = pl.items;
    launch_gather(a, p.kv_block, pl.kind == 2, s);
  }
  if (pl.kind != 1) {
    CombArgs c;
    c.part_o = part_o; c.part_ml = part_ml; c.cnt = cnt; c.items = pl.items;
    if (pl.kind == 0) { c.unit_num = p.kv_block; c.unit_den = pl.tok_per_item; c.qvc = 1; }
    else { c.unit_num = 1; c.unit_den = kSplitBlocks; c.qvc = kCombQV; }
    c.Hkv = pl.Hkv; c.G = pl.G; c.NQB = pl.NQB; c.q_block = p.q_block; c.Lq = pl.Lq; c.D = pl.D; c.QV = pl.qv;
    c.row_mask = row_mask; c.o = o.data; c.osb = o.stride_b; c.osh = o.stride_h; c.osl = o.stride_l; c.lse = lse;
    launch_combine(c, o.dtype, pl.B, s);
  }
}

}  // namespace bsa
