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
// K/V tiles are copied straight from global memory into LDS (double-buffered)
// and shared by the waves of a workgroup; each wave owns 32 query vectors.
// Online softmax in fp32 with exp2; the running max and sum are lane-local
// (see mfma_tile.cuh).
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

// One workgroup = NW waves of 32 query vectors.  Direct mode: NW / 4 heads of
// one KV group (4 waves of 32 rows each per head) share every K/V tile.  Split
// mode (NW = 4): the active (row, head) pairs of a query block, compacted.
// K/V tiles are double-buffered in LDS: the copy of tile u + 1 runs while
// tile u is computed, so one barrier per tile suffices.  A list entry (a KV
// block of SUB * KVB keys) is walked as SUB tiles of KVB keys: with 64-key
// tiles two workgroups fit on a CU and their waves overlap freely.
template <int KVB, int NW, bool SPLIT, int SUB = 1>
__global__ __launch_bounds__(NW * 64, (NW == 4 && KVB == 64) ? 2 : 1) void gather_mfma_kernel(GatherArgs a) {
  constexpr int TILE = KVB * kRow;                 // elements of one K or V tile
  constexpr int HPW = SPLIT ? 1 : NW / 4;          // heads per workgroup
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE];   // K0 V0 K1 V1
  __shared__ int qv_row[128], qv_head[128], qv_full[128];
  __shared__ int n_qv_sh;

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, g, qb, item = 0, h0 = 0;
  if (SPLIT) {
    item = blockIdx.x;
    qb = blockIdx.y;
    b = blockIdx.z / a.Hkv;
    g = blockIdx.z - b * a.Hkv;
  } else {
    // XCD-aware order: workgroup n runs on XCD n % 8; give each XCD a contiguous
    // run of (batch, group, query block descending, head set) work items.
    const int total = gridDim.x;
    const int n = blockIdx.x;
    const int i = (total % 8 == 0) ? (n % 8) * (total / 8) + n / 8 : n;
    const int sets = a.G / HPW;
    h0 = (i % sets) * HPW;
    const int rest = i / sets;
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
  const int wr = w & 3;                            // wave within its head
  const int qv = 32 * wr + r32;
  bool valid;
  int row, h;
  if (SPLIT) {
    valid = qv < n_qv;
    row = valid ? qv_row[qv] : 0;
    h = g * a.G + (valid ? qv_head[qv] : 0);
  } else {
    row = qb * a.q_block + qv;
    valid = qv < a.q_block && row < a.Lq;
    h = g * a.G + h0 + (w >> 2);
  }
  const bool wave_busy = SPLIT ? (32 * wr < n_qv) : (32 * wr < a.q_block && qb * a.q_block + 32 * wr < a.Lq);
  const int qpos = a.q_pos0 + row;
  // smallest query position of the wave (for deciding whether a tile needs the causal mask)
  int wave_min_pos = valid ? qpos : 0x7FFFFFFF;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_min_pos = min(wave_min_pos, wave_xor(wave_min_pos, m));

  bf16x8 qf[8];
  load_q_frag(a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)row * a.qsl, valid, qf);
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  const int32_t* list = a.idx + li * a.cap;
  // rows of tile u (of list entry e0 + u / SUB) inside the KV sequence (0 for
  // an index outside it, or a part beyond the end: nothing is read)
  auto entry_rows = [&](int u, int& key0) {
    const int j = list[e0 + u / SUB];
    const int blk0 = j * (KVB * SUB);
    key0 = blk0 + (u % SUB) * KVB;
    return (j < 0 || blk0 >= a.L || key0 >= a.L) ? 0 : min(KVB, a.L - key0);
  };
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int e, int buf) {
    int key0;
    const int nk = entry_rows(e, key0);
    if (nk == 0) return;
    issue_tile<KVB, NW>(kbg + (int64_t)key0 * a.ksl, a.ksl, nk, lds0 + (uint32_t)(buf * 2 * TILE * 2));
    issue_tile<KVB, NW>(vbg + (int64_t)key0 * a.vsl, a.vsl, nk, lds0 + (uint32_t)((buf * 2 + 1) * TILE * 2));
  };

  const int nt = (e1 - e0) * SUB;
  // largest query position of the wave: a tile wholly after it is skipped
  int wave_max_pos = valid ? qpos : -1;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_max_pos = max(wave_max_pos, wave_xor(wave_max_pos, m));
  wave_max_pos = __builtin_amdgcn_readfirstlane(wave_max_pos);
  if (nt > 0) issue(0, 0);
  for (int u = 0; u < nt; ++u) {
    const int buf = u & 1;
    int key0;
    const int nk = entry_rows(u, key0);
    wait_tile_loads();                             // this wave's part of tile u is in LDS
    __syncthreads();                               // ... and everyone's; tile u - 1 is finished
    if (u + 1 < nt) issue(u + 1, buf ^ 1);
    if (nk == 0 || !wave_busy || (a.causal && key0 > wave_max_pos)) continue;
    const uint16_t* Ks = lds + buf * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;
    f32x16 s[KVB / 32];
    qk_tile<KVB>(Ks, kofs, qf, s);
    const bool need_mask = nk < KVB || (a.causal && key0 + KVB - 1 > wave_min_pos);
    if (need_mask) {
      // largest visible key offset of this lane's query in the tile
      int lim = nk - 1;
      if (a.causal) lim = min(lim, qpos - key0);
      mask_tile<KVB / 32>(s, lim);
    }
    const float msub = softmax_rescale(tile_max<KVB / 32>(s) * a.c2, m_ref, l_run, o);
    softmax_pv_tile<KVB>(Vs, vofs, s, a.c2, msub, l_run, o);
  }

  if (!wave_busy) return;
  const float l_tot = pair_sum(l_run);
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
          l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
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
      a.part_ml[pi * 2] = m_ref;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

// Direct mode for an even group size: one workgroup = 8 waves = two heads of
// one KV group over a query block of up to 128 rows (waves 0-3 head h0 =
// group A, waves 4-7 head h0 + 1 = group B).  Waves w and w + 4 share a SIMD,
// so the two groups run half a list entry apart: while A computes S = K Q^T
// of entry e on the matrix cores, B runs the softmax and P V of entry e - 1,
// and the other way round in the next phase.  The vector-ALU softmax of one
// wave then overlaps the MFMA work of its partner instead of queueing behind
// the barriers that keep the groups in step.  K and V have two LDS buffers
// each; the K copy of entry e + 1 is issued once B has finished reading the
// K buffer it replaces (one phase after A did), the V copy likewise, so each
// copy has a whole entry of compute to land.
template <int KVB>
__global__ __launch_bounds__(512, 1) void gather_pp_kernel(GatherArgs a) {
  constexpr int NW = 8;
  constexpr int TILE = KVB * kRow;
  constexpr int IT = KVB / 4 / NW;                 // copy instructions per wave for one K or V tile
  // K buffers 0, 1 then V buffers 0, 1, always addressed with a compile-time
  // parity so that the LDS reads use immediate offsets.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE];
  __shared__ int list_sh[kMaxListMfma];

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: role branches stay scalar
  const int grp = w >> 2, wr = w & 3;
  // XCD-aware order: workgroup n runs on XCD n % 8; give each XCD a contiguous
  // run of (batch, group, query block descending, head pair) work items.
  const int total = gridDim.x, nb = blockIdx.x;
  const int wi = (total % 8 == 0) ? (nb % 8) * (total / 8) + nb / 8 : nb;
  const int sets = a.G / 2;
  const int h0 = (wi % sets) * 2;
  const int rest = wi / sets;
  const int qb = a.NQB - 1 - rest % a.NQB;
  const int bgi = rest / a.NQB;
  const int b = bgi / a.Hkv, g = bgi - b * a.Hkv;
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  const int n = min(a.cnt[li], a.cap);
  const int32_t* list = a.idx + li * a.cap;
  for (int i = tid; i < n; i += NW * 64) list_sh[i] = list[i];
  __syncthreads();

  const int h = g * a.G + h0 + grp;
  const int qv = 32 * wr + r32;
  const int row = qb * a.q_block + qv;
  const bool valid = qv < a.q_block && row < a.Lq;
  const bool wave_busy = 32 * wr < a.q_block && qb * a.q_block + 32 * wr < a.Lq;
  const int qpos = a.q_pos0 + row;
  int wave_min_pos = valid ? qpos : 0x7FFFFFFF;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_min_pos = min(wave_min_pos, wave_xor(wave_min_pos, m));
  wave_min_pos = __builtin_amdgcn_readfirstlane(wave_min_pos);

  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  const uint32_t kvoff = tile_lane_offset<NW>(a.ksl), vvoff = tile_lane_offset<NW>(a.vsl);
  // Copy K or V of list entry e into dst.  Always IT instructions per wave, so
  // the vmcnt bookkeeping below holds; an index outside the sequence copies
  // the first rows (the entry is then masked out entirely).
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int e, bool is_v, int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + (uint32_t)((is_v ? 2 + buf : buf) * TILE * 2);
    const int j = __builtin_amdgcn_readfirstlane(list_sh[e]);
    const int key0 = j * KVB;
    const bool ok = j >= 0 && key0 < a.L;
    const uint16_t* base = is_v ? vbg : kbg;
    const int64_t sl = is_v ? a.vsl : a.ksl;
    if (ok && key0 + KVB <= a.L)
      issue_full_tile<KVB, NW>(base + (int64_t)key0 * sl, sl, is_v ? vvoff : kvoff, dst);
    else
      issue_tile<KVB, NW>(base + (ok ? (int64_t)key0 * sl : 0), sl, ok ? a.L - key0 : min(KVB, a.L), dst);
  };
  bf16x8 qf[8];
  load_q_frag(a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)row * a.qsl, valid, qf);
  // Let the Q loads land before any tile copy is issued: a use of Q inside the
  // loop would otherwise wait on every copy in flight.
  settle(qf);
  if (n > 0) { issue(0, false, 0); issue(0, true, 0); }
  if (n > 1) { issue(1, false, 1); issue(1, true, 1); }
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 s[KVB / 32];

  auto smpv = [&](int e, const uint16_t* Vs) __attribute__((always_inline)) {
    const int j = __builtin_amdgcn_readfirstlane(list_sh[e]);
    const int key0 = j * KVB;
    const int nk = (j < 0 || key0 >= a.L) ? 0 : min(KVB, a.L - key0);
    if (nk < KVB || (a.causal && key0 + KVB - 1 > wave_min_pos)) {
      int lim = nk - 1;                            // largest visible key offset of this lane's query
      if (a.causal) lim = min(lim, qpos - key0);
      mask_tile<KVB / 32>(s, lim);
    }
    const float msub = softmax_rescale(tile_max<KVB / 32>(s) * a.c2, m_run, l_run, o);
    softmax_pv_tile<KVB>(Vs, vofs, s, a.c2, msub, l_run, o);
  };

  // Entry t lives in the buffers of parity t & 1; the copies of entry t + 1
  // go to the other ones.  Both roles pass the same two barriers per entry.
  auto sync_k = [&](int t) __attribute__((always_inline)) {
    // K of entry t must be in LDS: the copies issued after it (V of t, and at
    // the start K and V of entry 1) may still be in flight
    if (t == 0 && n > 1) wait_loads_but<3 * IT>();
    else wait_loads_but<IT>();
    lds_barrier();                                 // ... for every wave; B is done with the K buffer of t - 1
    if (t >= 1 && t + 1 < n) issue(t + 1, false, (t + 1) & 1);
  };
  auto sync_v = [&](int t) __attribute__((always_inline)) {
    // V of entry t must be in LDS: only the K copy of entry t + 1 (or at the
    // start K and V of entry 1) may still be in flight
    if (t == 0) {
      if (n > 1) wait_loads_but<2 * IT>();
      else wait_loads_but<0>();
    } else if (t + 1 < n) {
      wait_loads_but<IT>();
    } else {
      wait_loads_but<0>();
    }
    lds_barrier();                                 // ... for every wave; B is done with the V buffer of t - 1
    if (t >= 1 && t + 1 < n) issue(t + 1, true, (t + 1) & 1);
  };
  if (grp == 0) {                                  // A: K Q^T of t, then softmax + P V of t
    for (int t = 0; t < n; ++t) {
      sync_k(t);
      if (wave_busy) qk_tile<KVB>(lds + (t & 1) * TILE, kofs, qf, s);
      sync_v(t);
      if (wave_busy) smpv(t, lds + (2 + (t & 1)) * TILE);
    }
  } else {                                         // B: softmax + P V of t - 1, then K Q^T of t
    for (int t = 0; t < n; ++t) {
      sync_k(t);
      if (wave_busy && t >= 1) smpv(t - 1, lds + (2 + ((t - 1) & 1)) * TILE);
      sync_v(t);
      if (wave_busy) qk_tile<KVB>(lds + (t & 1) * TILE, kofs, qf, s);
    }
    if (wave_busy && n > 0) smpv(n - 1, lds + (2 + ((n - 1) & 1)) * TILE);
  }

  if (!wave_busy || !valid) return;
  const float l_tot = pair_sum(l_run);
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
    a.lse[((int64_t)b * a.Hkv * a.G + h) * a.Lq + row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

void launch_gather(const GatherArgs& a, int kv_block, bool split, hipStream_t s) {
  if (split) {
    dim3 grid(a.items, a.NQB, a.B * a.Hkv);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<128, 4, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, 4, true>), grid, dim3(256), 0, s, a);
  } else if (a.G % 2 == 0) {
    dim3 grid(a.B * a.Hkv * a.NQB * (a.G / 2));
    if (kv_block == 128) hipLaunchKernelGGL((gather_pp_kernel<128>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gather_pp_kernel<64>), grid, dim3(512), 0, s, a);
  } else {
    // odd group size: one head per workgroup, 64-key tiles (two workgroups per CU)
    dim3 grid(a.B * a.Hkv * a.NQB * a.G);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<64, 4, false, 2>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, 4, false>), grid, dim3(256), 0, s, a);
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
    if (pl.kind == 0) { c.unit_num = p.kv_block; c.unit_den = pl.tok_per_item; }
    else { c.unit_num = 1; c.unit_den = kSplitBlocks; }
    c.qvc = 256 / pl.D;                          // one thread per (query vector, dim)
    c.Hkv = pl.Hkv; c.G = pl.G; c.NQB = pl.NQB; c.q_block = p.q_block; c.Lq = pl.Lq; c.D = pl.D; c.QV = pl.qv;
    c.row_mask = row_mask; c.o = o.data; c.osb = o.stride_b; c.osh = o.stride_h; c.osl = o.stride_l; c.lse = lse;
    launch_combine(c, o.dtype, pl.B, s);
  }
}

}  // namespace bsa
