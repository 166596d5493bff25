// Merge of two attention states over disjoint key sets (LoSA page, technical
// summary sec. 2: a stable token reuses the prefix-attention output and
// statistics of the previous step; its attention over the whole context is
// that cached prefix state combined with the state over the block's own keys).
//
// With O_x the softmax-weighted mean of V over key set x and lse_x the natural
// log of its softmax denominator, the state over the union of the two sets is
//   lse = ln(e^lse_a + e^lse_b),  O = (e^(lse_a - lse) O_a + e^(lse_b - lse) O_b).
// An lse of -inf is an empty set (weight 0).
//
// One wave per (batch, head, row), each lane a fixed set of dims: elementwise
// over HBM, every element read once and written once.
#include "common.h"
#include "internal.h"
#include "mfma_tile.h"
#include "split.h"

namespace bsa {

template <int DA, int DB, int DO>
__global__ __launch_bounds__(256) void merge_states_kernel(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const int64_t l = row % a.L, bh = row / a.L;
  const int64_t h = bh % a.H, b = bh / a.H;
  const float la = a.lse_a[row], lb = a.lse_b[row];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m > -INFINITY) {
    wa = la > -INFINITY ? fast_exp2((la - m) * kLog2e) : 0.f;
    wb = lb > -INFINITY ? fast_exp2((lb - m) * kLog2e) : 0.f;
    const float s = wa + wb;                         // >= 1: the larger weight is exactly 1
    lse = m + log2f(s) * kLn2;
    wa /= s;
    wb /= s;
  }
  const int64_t ia = b * a.asb + h * a.ash + l * a.asl, ib = b * a.bsb + h * a.bsh + l * a.bsl;
  const int64_t io = b * a.osb + h * a.osh + l * a.osl;
  for (int d = 2 * lane; d < a.D; d += 128) {
    float xa[2], xb[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      xa[e] = DA == BSA_BF16 ? bf16lo((uint32_t)reinterpret_cast<const uint16_t*>(a.o_a)[ia + d + e])
                             : reinterpret_cast<const float*>(a.o_a)[ia + d + e];
      xb[e] = DB == BSA_BF16 ? bf16lo((uint32_t)reinterpret_cast<const uint16_t*>(a.o_b)[ib + d + e])
                             : reinterpret_cast<const float*>(a.o_b)[ib + d + e];
    }
    // an empty side contributes nothing, whatever its O holds
    const float y0 = (wa > 0.f ? wa * xa[0] : 0.f) + (wb > 0.f ? wb * xb[0] : 0.f);
    const float y1 = (wa > 0.f ? wa * xa[1] : 0.f) + (wb > 0.f ? wb * xb[1] : 0.f);
    if (DO == BSA_BF16) reinterpret_cast<uint32_t*>(a.o)[(io + d) / 2] = pack_bf16x2(y0, y1);
    else *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(a.o) + io + d) = f32x2{y0, y1};
  }
  if (lane == 0) a.lse[row] = lse;
}

void launch_merge_states(const MergeArgs& a, int da, int db, int dout, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + 3) / 4));
#define BSA_MERGE(A, B_, O) hipLaunchKernelGGL((merge_states_kernel<A, B_, O>), grid, dim3(256), 0, s, a)
#define BSA_MERGE_O(A, B_)                              \
  if (dout == BSA_BF16) BSA_MERGE(A, B_, BSA_BF16);     \
  else BSA_MERGE(A, B_, BSA_F32)
  if (da == BSA_BF16) {
    if (db == BSA_BF16) { BSA_MERGE_O(BSA_BF16, BSA_BF16); }
    else { BSA_MERGE_O(BSA_BF16, BSA_F32); }
  } else {
    if (db == BSA_BF16) { BSA_MERGE_O(BSA_F32, BSA_BF16); }
    else { BSA_MERGE_O(BSA_F32, BSA_F32); }
  }
#undef BSA_MERGE_O
#undef BSA_MERGE
}

}  // namespace bsa

namespace bsa {

// Attention of a denoising block's rows over the block's own keys (both
// directions: a block-wise diffusion LM denoises all tokens of a block
// together), merged with each row's cached prefix state -- one kernel per
// step instead of a gather, its combine and a merge.
//
// One wave per (batch, query head): the R <= 32 rows are one 32-query tile and
// the block's keys one 32-key tile, so the step is one tile of the MFMA
// attention (S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16, K
// and V copied straight into LDS, the tile's max as the softmax reference).
// The copies, the query fragments and the row's cached prefix (O, lse) are
// all requested before the first product.
// The requests of one wave's block tile: the K and V tiles into LDS, the
// query fragments of lane row r32 (rows past R load row R - 1 and are zeroed)
// and that row's cached prefix state (O in the O^T layout: dims
// 32 dt + 8 i4 + 4 hi .. + 3, and its lse).  Returns the lane's row.  Run by
// wave 0 of its workgroup: the tile copies place LDS rows by wave index.
template <bool PRE_F32>
__device__ __forceinline__ int block_tile_requests(const BlockMergeArgs& a, int b, int h, uint32_t l0, bf16x8 (&qf)[8],
                                                   float (&op)[4][4][4], float& la) {
  constexpr int KVB = 32;
  const int g = h / a.G, lane = threadIdx.x & 63, r32 = lane & 31, hi = lane >> 5;
  const int R = a.R;
  // rows past R repeat row R - 1: their keys are masked and their V rows weighted by zero
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.kb);
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.vb);
  issue_tile<KVB, 1>(kb + (int64_t)b * a.ksb + (int64_t)g * a.ksh, a.ksl, R, l0);
  issue_tile<KVB, 1>(vb + (int64_t)b * a.vsb + (int64_t)g * a.vsh, a.vsl, R, l0 + KVB * kRow * 2);
  const int row = min(r32, R - 1);
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)b * a.qsb + (int64_t)h * a.qsh +
                           (int64_t)row * a.qsl;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hi);
  }
  {
    const int64_t io = (int64_t)b * a.psb + (int64_t)h * a.psh + (int64_t)row * a.psl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * dt + 8 * i4 + 4 * hi;
        if constexpr (PRE_F32) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.o_pre) + io + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) op[dt][i4][e] = x[e];
        } else {
          const u32x2 x = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(a.o_pre) + io + d);
          op[dt][i4][0] = bf16lo(x[0]);
          op[dt][i4][1] = bf16hi(x[0]);
          op[dt][i4][2] = bf16lo(x[1]);
          op[dt][i4][3] = bf16hi(x[1]);
        }
      }
  }
  la = a.lse_pre[((int64_t)b * a.Hq + h) * R + row];
  if (r32 >= R) {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bf16x8{};
  }
  return row;
}

// The block tile once its inputs are in LDS: S^T = K Q^T masked to the R
// keys, softmax with the tile's max, O^T = V^T P^T; returns the block part's
// lse (natural log) and leaves its unnormalised O and row sum in o / l_tot.
__device__ __forceinline__ float block_tile_compute(const BlockMergeArgs& a, const uint16_t* lds,
                                                    const bf16x8 (&qf)[8], f32x16 (&o)[4], float& l_tot) {
  constexpr int KVB = 32;
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);
  wait_tile_loads();                                 // the tiles are in LDS (one wave: no barrier)
  const float c2 = a.scale * kLog2e;
  f32x16 s[1];
  qk_tile<KVB>(lds, kofs, qf, s);
  mask_tile<1>(s, a.R - 1);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;
  const float msub = softmax_rescale(tile_max<1>(s) * c2, m_ref, l_run, o);
  softmax_pv_tile<KVB>(lds + KVB * kRow, vofs, s, c2, msub, l_run, o);
  l_tot = pair_sum(l_run);
  return (m_ref + log2f(l_tot)) * kLn2;             // >= 1 key
}

// O and lse of lane row `row` from the prefix state (op, la) and the block part (o, lb, l_tot).
template <int DO>
__device__ __forceinline__ void block_merge_store(const BlockMergeArgs& a, int b, int h, int row,
                                                  const float (&op)[4][4][4], float la, const f32x16 (&o)[4], float lb,
                                                  float l_tot) {
  const int hi = (threadIdx.x & 63) >> 5;
  const float m = fmaxf(la, lb);
  const float wa = la > -INFINITY ? fast_exp2((la - m) * kLog2e) : 0.f;
  const float wb = fast_exp2((lb - m) * kLog2e);
  const float tot = wa + wb;
  const float ca = wa / tot, cb = wb / (tot * l_tot);
  const int64_t io = (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)row * a.osl;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * dt + 8 * i4 + 4 * hi;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (wa > 0.f ? ca * op[dt][i4][e] : 0.f) + cb * o[dt][4 * i4 + e];
      if (DO == BSA_BF16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + io + d) =
            u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + io + d) = f32x4{y[0], y[1], y[2], y[3]};
      }
    }
  if (hi == 0) a.lse[((int64_t)b * a.Hq + h) * a.R + row] = m + log2f(tot) * kLn2;
}

// One wave per (batch, query head): the R <= 32 rows are one 32-query tile and
// the block's keys one 32-key tile, so the step is one tile of the MFMA
// attention (S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16, K
// and V copied straight into LDS, the tile's max as the softmax reference).
// The copies, the query fragments and the row's cached prefix (O, lse) are
// all requested before the first product.
template <int DO, bool PRE_F32>
__global__ __launch_bounds__(64) void block_attn_merge_kernel(BlockMergeArgs a) {
  constexpr int KVB = 32;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * KVB * kRow];   // K tile, then V tile
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  bf16x8 qf[8];
  float op[4][4][4], la;
  const int row = block_tile_requests<PRE_F32>(a, b, h, lds_addr(lds), qf, op, la);
  f32x16 o[4];
  float l_tot;
  const float lb = block_tile_compute(a, lds, qf, o, l_tot);
  if ((int)(threadIdx.x & 31) >= a.R) return;
  block_merge_store<DO>(a, b, h, row, op, la, o, lb, l_tot);
}

// ------------------------------------------------------- denoising step ---
// The last launch of the fused denoising step: the combine of the split
// partials of the active rows (the prefix attention over the block's list;
// written to the prefix cache, as the combine of the attention entry point
// writes O and LSE), then the block tile and the merge of every row, as the
// block-merge entry point.  One workgroup of five waves per (kDenRows rows,
// batch, query head): wave 1 + r combines row r0 + r (two dims per lane,
// partial slices in batches of 32 with a running maximum, the combine's
// arithmetic; a stable row's wave has nothing to do), while wave 0 (the tile
// copies address LDS rows by wave index) copies the block's K/V tile,
// computes the block tile for all rows and then, once the combined prefix of
// the active rows is in LDS, merges and writes its rows.
template <int DO>
__global__ __launch_bounds__(320) void den_merge_kernel(DenMergeArgs a) {
  constexpr int KVB = 32, BATCH = 32, RC = kDenRows;
  static_assert(RC == 4, "one combining wave per row");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * KVB * kRow];
  __shared__ __attribute__((aligned(16))) uint64_t ml_sh[RC][2 * BATCH];
  __shared__ __attribute__((aligned(16))) float pre_sh[RC][kD];
  __shared__ float pre_lse_sh[RC];
  const BlockMergeArgs& m = a.m;
  const int r0 = blockIdx.x * RC, bh = blockIdx.y;
  const int b = bh / m.Hq, h = bh - b * m.Hq, g = h / m.G, hl = h - g * m.G;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int R = m.R;
  if (w == 0) {
    // ---- wave 0: the block tile, then (after the combine) the merge
    bf16x8 qf[8];
    float op[4][4][4], la;
    const int trow = block_tile_requests<true>(m, b, h, lds_addr(lds), qf, op, la);
    const uint8_t tact = a.row_mask[(int64_t)b * R + trow];
    f32x16 o[4];
    float l_tot;
    const float lb = block_tile_compute(m, lds, qf, o, l_tot);
    __syncthreads();                                        // the combined prefixes are in LDS
    const int r32 = lane & 31;
    if (r32 >= R || r32 < r0 || r32 >= r0 + RC) return;
    if (tact) {
      // an active row's prefix is the one just combined (the values written to the cache)
      const int hi = lane >> 5;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&pre_sh[r32 - r0][32 * dt + 8 * i4 + 4 * hi]);
#pragma unroll
          for (int e = 0; e < 4; ++e) op[dt][i4][e] = x[e];
        }
      la = pre_lse_sh[r32 - r0];
    }
    block_merge_store<DO>(m, b, h, trow, op, la, o, lb, l_tot);
    return;
  }
  // ---- waves 1..4: the combine of row r0 + rl (dims 2 lane, + 1)
  const int rl = w - 1, d = 2 * lane;
  const int row = r0 + rl, rowc = min(row, R - 1);
  const uint8_t rbyte = (uint8_t)__builtin_amdgcn_readfirstlane(a.row_mask[(int64_t)b * R + rowc]);
  const int64_t li = (int64_t)b * a.Hkv + g;
  const int c_list = a.cnt[li];
  const int QV = R * m.G, qv = rowc * m.G + hl;
  const int64_t p0 = li * a.items;
  const int per = split_per(c_list, a.items);
  const int nvalid = (c_list + per - 1) / per;
  const bool live = row < R && rbyte != 0;                  // uniform over the wave
  if (live) {
    float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
    // one batch of 32 slices: a running maximum, then the slices in order (the combine's arithmetic)
    auto batch = [&](int it0, const float (&o0)[BATCH], const float (&o1)[BATCH], const uint64_t* mls)
        __attribute__((always_inline)) {
      uint64_t mlr[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH / 2; ++q) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(mls + 2 * q);
        mlr[2 * q] = (uint64_t)t[0] | ((uint64_t)t[1] << 32);
        mlr[2 * q + 1] = (uint64_t)t[2] | ((uint64_t)t[3] << 32);
      }
      float bm = M;
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (it0 + u < nvalid) bm = fmaxf(bm, __uint_as_float((uint32_t)mlr[u]));
      if (bm != -INFINITY) {                                // else nothing visible so far
        const float alpha = M == -INFINITY ? 0.f : fast_exp2(M - bm);
        L *= alpha;
        acc0 *= alpha;
        acc1 *= alpha;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const float mv = __uint_as_float((uint32_t)mlr[u]);
          // selects, not a branch per slice (a skipped slot's stale values are never multiplied in)
          const bool use = it0 + u < nvalid && mv != -INFINITY;
          const float wgt = fast_exp2(mv - bm);
          const float l2 = fmaf(__uint_as_float((uint32_t)(mlr[u] >> 32)), wgt, L);
          const float a0 = fmaf(o0[u], wgt, acc0), a1 = fmaf(o1[u], wgt, acc1);
          L = use ? l2 : L;
          acc0 = use ? a0 : acc0;
          acc1 = use ? a1 : acc1;
        }
        M = bm;
      }
    };
    // two batches are requested together (their loads overlap; the arithmetic stays per batch)
    for (int it0 = 0; it0 < nvalid; it0 += 2 * BATCH) {
      // slots past the valid count are clamped to a written one and excluded in batch()
      const int64_t itm = min(it0 + lane, nvalid - 1);
      const uint64_t mlv = *reinterpret_cast<const uint64_t*>(a.part_ml + ((p0 + itm) * QV + qv) * 2);
      float oa0[BATCH], oa1[BATCH], ob0[BATCH], ob1[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t it = min(it0 + u, nvalid - 1);
        const f32x2 v = *reinterpret_cast<const f32x2*>(a.part_o + ((p0 + it) * QV + qv) * kD + d);
        oa0[u] = v[0];
        oa1[u] = v[1];
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t it = min(it0 + BATCH + u, nvalid - 1);
        const f32x2 v = *reinterpret_cast<const f32x2*>(a.part_o + ((p0 + it) * QV + qv) * kD + d);
        ob0[u] = v[0];
        ob1[u] = v[1];
      }
      ml_sh[rl][lane] = mlv;
      wave_sync_lds();
      batch(it0, oa0, oa1, &ml_sh[rl][0]);
      if (it0 + BATCH < nvalid) batch(it0 + BATCH, ob0, ob1, &ml_sh[rl][BATCH]);
      wave_sync_lds();                                      // read before the next pair rewrites it
    }
    const float y0 = L > 0.f ? acc0 / L : 0.f, y1 = L > 0.f ? acc1 / L : 0.f;
    const float lp = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    float* co = a.cache_o + (int64_t)b * m.psb + (int64_t)h * m.psh + (int64_t)row * m.psl + d;
    *reinterpret_cast<f32x2*>(co) = f32x2{y0, y1};
    pre_sh[rl][d] = y0;
    pre_sh[rl][d + 1] = y1;
    if (lane == 0) {
      a.cache_lse[((int64_t)b * m.Hq + h) * R + row] = lp;
      pre_lse_sh[rl] = lp;
    }
  }
  __syncthreads();
}

void launch_den_merge(const DenMergeArgs& a, int dout, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(a.m.R, kDenRows), (unsigned)(a.m.B * a.m.Hq));
  if (dout == BSA_BF16) hipLaunchKernelGGL((den_merge_kernel<BSA_BF16>), grid, dim3(64 * (kDenRows + 1)), 0, s, a);
  else hipLaunchKernelGGL((den_merge_kernel<BSA_F32>), grid, dim3(64 * (kDenRows + 1)), 0, s, a);
}

void launch_block_attn_merge(const BlockMergeArgs& a, int dout, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.Hq));
  if (dout == BSA_BF16) {
    if (a.pre_f32) hipLaunchKernelGGL((block_attn_merge_kernel<BSA_BF16, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((block_attn_merge_kernel<BSA_BF16, false>), grid, dim3(64), 0, s, a);
  } else {
    if (a.pre_f32) hipLaunchKernelGGL((block_attn_merge_kernel<BSA_F32, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((block_attn_merge_kernel<BSA_F32, false>), grid, dim3(64), 0, s, a);
  }
}

}  // namespace bsa
