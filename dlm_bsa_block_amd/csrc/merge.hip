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
template <int DO, bool PRE_F32>
__global__ __launch_bounds__(64) void block_attn_merge_kernel(BlockMergeArgs a) {
  constexpr int KVB = 32;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * KVB * kRow];   // K tile, then V tile
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  const int lane = threadIdx.x, r32 = lane & 31, hi = lane >> 5;
  const int R = a.R;
  const uint32_t l0 = lds_addr(lds);
  // rows past R repeat row R - 1: their keys are masked and their V rows weighted by zero
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.kb);
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.vb);
  issue_tile<KVB, 1>(kb + (int64_t)b * a.ksb + (int64_t)g * a.ksh, a.ksl, R, l0);
  issue_tile<KVB, 1>(vb + (int64_t)b * a.vsb + (int64_t)g * a.vsh, a.vsl, R, l0 + KVB * kRow * 2);
  // this lane's query row (rows past R load row R - 1 and are zeroed)
  const bool valid = r32 < R;
  const int row = min(r32, R - 1);
  bf16x8 qf[8];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)b * a.qsb + (int64_t)h * a.qsh +
                           (int64_t)row * a.qsl;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hi);
  }
  // the row's cached prefix state, in the O^T layout: dims 32 dt + 8 i4 + 4 hi .. + 3
  float op[4][4][4];
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
  const float la = a.lse_pre[((int64_t)b * a.Hq + h) * R + row];
  if (!valid) {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bf16x8{};
  }
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);
  wait_tile_loads();                                 // the tiles are in LDS (one wave: no barrier)

  const float c2 = a.scale * kLog2e;
  f32x16 s[1];
  qk_tile<KVB>(lds, kofs, qf, s);
  mask_tile<1>(s, R - 1);
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;
  const float msub = softmax_rescale(tile_max<1>(s) * c2, m_ref, l_run, o);
  softmax_pv_tile<KVB>(lds + KVB * kRow, vofs, s, c2, msub, l_run, o);
  const float l_tot = pair_sum(l_run);

  if (!valid) return;
  const float lb = (m_ref + log2f(l_tot)) * kLn2;   // the block part's lse (natural log); >= 1 key
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
  if (hi == 0) a.lse[((int64_t)b * a.Hq + h) * R + row] = m + log2f(tot) * kLn2;
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
