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
// One workgroup per (batch, query head), four waves, each wave eight rows.
// Round trip one brings q, the group's block keys and values and the row's
// cached prefix (O, lse).  S = scale q k^T: lane (j, half) sums its half of the
// dims for key j, then the halves are added across lanes l and l ^ 32; the
// softmax over the R keys reduces over 32-lane halves (DPP and a lane swap);
// P goes to LDS, and O = P V takes each lane over two dims.  All in fp32.
// max / sum over each 32-lane half of the wave (DPP inside 16-lane rows, then
// the row pair through v_permlane16_swap); every lane of a half gets the same bits
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(-INFINITY, v));         // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(-INFINITY, v));         // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(-INFINITY, v));        // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(-INFINITY, v));        // row_mirror
  float lo, hi;
  lane_pair16(v, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_sum(float v) {
  v = group_sum<16>(v);
  float lo, hi;
  lane_pair16(v, lo, hi);
  return lo + hi;
}

template <int DO, bool PRE_F32>
__global__ __launch_bounds__(256) void block_attn_merge_kernel(BlockMergeArgs a) {
  constexpr int D = 128, MAXR = 32, RW = MAXR / 4;   // rows per wave
  constexpr int KP = D + 4;                          // padded key rows: 16-byte reads, lanes spread over banks
  __shared__ __align__(16) float qs[MAXR][D];
  __shared__ __align__(16) float ks[MAXR][KP];
  __shared__ __align__(16) float vs[MAXR][D];
  __shared__ __align__(16) float ps[MAXR][MAXR + 4];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq, g = h / a.G;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int R = a.R;
  const int j = lane & 31, half = lane >> 5;
  const int d0 = 2 * lane;                           // this lane's two dims in P V and the merge

  // ---- round trip 1: q, kb, vb (bf16) into LDS as f32; the cached prefix state into registers
  float op[RW][2], lp[RW];
  {
    u32x4 qv[2], kv[2], vv[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = (tid + 256 * it) * 8;            // element index in an R x D tile
      const int r = min(e / D, R - 1), d = e % D;
      qv[it] = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)r * a.qsl + d) * 2);
      kv[it] = *reinterpret_cast<const u32x4*>(a.kb + ((int64_t)b * a.ksb + (int64_t)g * a.ksh + (int64_t)r * a.ksl + d) * 2);
      vv[it] = *reinterpret_cast<const u32x4*>(a.vb + ((int64_t)b * a.vsb + (int64_t)g * a.vsh + (int64_t)r * a.vsl + d) * 2);
    }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const int r = min(w * RW + rr, R - 1);
      const int64_t io = (int64_t)b * a.psb + (int64_t)h * a.psh + (int64_t)r * a.psl + d0;
      // the cached state's dtype is a template argument: a branch around these loads would make
      // each row's load wait for the previous one
      if constexpr (PRE_F32) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(reinterpret_cast<const float*>(a.o_pre) + io);
        op[rr][0] = x[0];
        op[rr][1] = x[1];
      } else {
        const uint32_t x = reinterpret_cast<const uint32_t*>(a.o_pre)[io / 2];
        op[rr][0] = bf16lo(x);
        op[rr][1] = bf16hi(x);
      }
      lp[rr] = a.lse_pre[((int64_t)b * a.Hq + h) * R + r];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = (tid + 256 * it) * 8;
      const int r = e / D, d = e % D;
      if (r < R) {
        f32x4 x0 = {bf16lo(qv[it][0]), bf16hi(qv[it][0]), bf16lo(qv[it][1]), bf16hi(qv[it][1])};
        f32x4 x1 = {bf16lo(qv[it][2]), bf16hi(qv[it][2]), bf16lo(qv[it][3]), bf16hi(qv[it][3])};
        *reinterpret_cast<f32x4*>(&qs[r][d]) = x0;
        *reinterpret_cast<f32x4*>(&qs[r][d + 4]) = x1;
        x0 = f32x4{bf16lo(kv[it][0]), bf16hi(kv[it][0]), bf16lo(kv[it][1]), bf16hi(kv[it][1])};
        x1 = f32x4{bf16lo(kv[it][2]), bf16hi(kv[it][2]), bf16lo(kv[it][3]), bf16hi(kv[it][3])};
        *reinterpret_cast<f32x4*>(&ks[r][d]) = x0;
        *reinterpret_cast<f32x4*>(&ks[r][d + 4]) = x1;
        x0 = f32x4{bf16lo(vv[it][0]), bf16hi(vv[it][0]), bf16lo(vv[it][1]), bf16hi(vv[it][1])};
        x1 = f32x4{bf16lo(vv[it][2]), bf16hi(vv[it][2]), bf16lo(vv[it][3]), bf16hi(vv[it][3])};
        *reinterpret_cast<f32x4*>(&vs[r][d]) = x0;
        *reinterpret_cast<f32x4*>(&vs[r][d + 4]) = x1;
      }
    }
  }
  __syncthreads();

  // ---- S = scale q k^T: lane (j, half) over dims [64 half, 64 half + 64), 4 dims per read
  float s[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) s[rr] = 0.f;
#pragma unroll 4
  for (int dd = 0; dd < D / 2; dd += 4) {
    const int d = half * (D / 2) + dd;
    const f32x4 kx = *reinterpret_cast<const f32x4*>(&ks[j][d]);
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const f32x4 qx = *reinterpret_cast<const f32x4*>(&qs[w * RW + rr][d]);
      s[rr] = fmaf(qx[0], kx[0], s[rr]);
      s[rr] = fmaf(qx[1], kx[1], s[rr]);
      s[rr] = fmaf(qx[2], kx[2], s[rr]);
      s[rr] = fmaf(qx[3], kx[3], s[rr]);
    }
  }
  // ---- softmax over the keys (both halves end with the same values)
  float mrow[RW], lrow[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    float x = pair_sum(s[rr]) * a.scale;
    x = j < R ? x : -INFINITY;
    const float m = half_max(x);
    const float p = j < R ? fast_exp2((x - m) * kLog2e) : 0.f;
    mrow[rr] = m;
    lrow[rr] = half_sum(p);
    if (half == 0) ps[w * RW + rr][j] = p;
  }
  __syncthreads();

  // ---- O = P V over the block's keys, then the merge with the prefix state
  float o[RW][2];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) o[rr][0] = o[rr][1] = 0.f;
  for (int j0 = 0; j0 < R; j0 += 4) {                // keys past R have p = 0 (ps holds zeros there)
    f32x2 vx[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vx[c] = *reinterpret_cast<const f32x2*>(&vs[min(j0 + c, R - 1)][d0]);
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(&ps[w * RW + rr][j0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[rr][0] = fmaf(p4[c], vx[c][0], o[rr][0]);
        o[rr][1] = fmaf(p4[c], vx[c][1], o[rr][1]);
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int r = w * RW + rr;
    if (r >= R) break;                               // uniform over the wave
    const float lb = mrow[rr] + log2f(lrow[rr]) * kLn2;   // the block part's lse (natural log)
    const float la = lp[rr];
    const float m = fmaxf(la, lb);                   // lb is finite: the block has at least one key
    const float wa = la > -INFINITY ? fast_exp2((la - m) * kLog2e) : 0.f;
    const float wb = fast_exp2((lb - m) * kLog2e);
    const float tot = wa + wb;
    const float ca = wa / tot, cb = wb / (tot * lrow[rr]);
    const float y0 = (wa > 0.f ? ca * op[rr][0] : 0.f) + cb * o[rr][0];
    const float y1 = (wa > 0.f ? ca * op[rr][1] : 0.f) + cb * o[rr][1];
    const int64_t io = (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)r * a.osl + d0;
    if (DO == BSA_BF16) reinterpret_cast<uint32_t*>(a.o)[io / 2] = pack_bf16x2(y0, y1);
    else *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(a.o) + io) = f32x2{y0, y1};
    if (lane == 0) a.lse[((int64_t)b * a.Hq + h) * R + r] = m + log2f(tot) * kLn2;
  }
}

void launch_block_attn_merge(const BlockMergeArgs& a, int dout, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.Hq));
  if (dout == BSA_BF16) {
    if (a.pre_f32) hipLaunchKernelGGL((block_attn_merge_kernel<BSA_BF16, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((block_attn_merge_kernel<BSA_BF16, false>), grid, dim3(256), 0, s, a);
  } else {
    if (a.pre_f32) hipLaunchKernelGGL((block_attn_merge_kernel<BSA_F32, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((block_attn_merge_kernel<BSA_F32, false>), grid, dim3(256), 0, s, a);
  }
}

}  // namespace bsa
