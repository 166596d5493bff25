// Softmax-threshold attention (BLASST page, technical summary sec. 2): inside
// the blockwise online softmax, a KV tile whose max logit trails the running
// row max by more than ln(1/lambda) is skipped -- no exponentials, no V load
// from HBM and no PV product.  The test reuses statistics the online softmax
// computes anyway.
//
// One workgroup per (query tile of 128 rows, pair of query heads of one KV
// group -- one head when the group size is odd); 4 waves of 32 rows per head.
// KV tiles are visited from the diagonal (the newest visible tile) down to
// tile 0.  For each tile S = K Q^T is always computed (the max needs it); each
// wave votes through a ballot, the votes of a head meet in LDS, and all waves
// of that head take the same keep/skip branch.  V is loaded only when a head
// of the workgroup keeps the tile, and its copy is issued before the
// exponentials so their latency overlaps it.  The K tile of the next step is
// copied into a second LDS buffer while the current one is used.  Workgroups
// of one KV group run on one XCD (heads of a query tile adjacent), so K/V
// tiles are shared through that XCD's L2.
#include <cmath>

#include "internal.h"
#include "mfma_tile.h"

namespace bsa {

struct ThrArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl;
  int B, Hkv, G, L, Lq, NQT, NKT, causal;
  float c2;        // scale * log2(e)
  float lnlam2;    // ln(lambda) * log2(e); -inf when lambda = 0
  void* o;                        // bf16, or f32 when o_f32
  int o_f32;
  int64_t osb, osh, osl;
  float* lse;
  int32_t* kept;
  uint8_t* keep_map;
};

constexpr int kTile = 128;

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void threshold_kernel(ThrArgs a) {
  constexpr int TILE = kTile * kRow;
  constexpr int HPW = NW / 4;                      // heads per workgroup (4 waves of 32 rows each)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * TILE];   // K0 K1 V
  __shared__ int flags[NW];

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keep/skip branches stay scalar
  const int wr = w & 3, hh = w >> 2;
  const int total = gridDim.x, n = blockIdx.x;
  const int wi = (total % 8 == 0) ? (n % 8) * (total / 8) + n / 8 : n;
  const int sets = a.G / HPW;
  const int h0 = (wi % sets) * HPW;
  const int rest = wi / sets;
  const int qt = a.NQT - 1 - rest % a.NQT;
  const int bgi = rest / a.NQT;
  const int b = bgi / a.Hkv, g = bgi - b * a.Hkv;
  const int h = g * a.G + h0 + hh;
  const int Hq = a.Hkv * a.G;

  const int row = qt * kTile + 32 * wr + r32;
  const bool valid = row < a.Lq;
  const bool wave_busy = qt * kTile + 32 * wr < a.Lq;
  int wave_min_pos = valid ? row : 0x7FFFFFFF;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_min_pos = min(wave_min_pos, wave_xor(wave_min_pos, m));
  const int last_row = min(a.Lq, (qt + 1) * kTile) - 1;
  const int jmax = a.causal ? min(a.NKT - 1, last_row / kTile) : a.NKT - 1;

  bf16x8 qf[8];
  load_q_frag(a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)min(row, a.Lq - 1) * a.qsl, valid, qf);
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;            // running max of the kept tiles (log2 units) and sum
  int nkept = 0;
  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  uint8_t* kmap = a.keep_map ? a.keep_map + (((int64_t)b * Hq + h) * a.NQT + qt) * a.NKT : nullptr;
  uint16_t* Vs = lds + 2 * TILE;

  const uint32_t lds0 = lds_addr(lds);
  issue_tile<kTile, NW>(kbg + (int64_t)jmax * kTile * a.ksl, a.ksl, min(kTile, a.L - jmax * kTile), lds0);
  for (int j = jmax, t = 0; j >= 0; --j, ++t) {
    const int key0 = j * kTile;
    const int nk = min(kTile, a.L - key0);
    const uint16_t* Ks = lds + (t & 1) * TILE;
    wait_tile_loads();                             // K of tile j (this wave's part)
    __syncthreads();                               // K visible; tile j + 1 finished (its K buffer and V free)
    if (j > 0)
      issue_tile<kTile, NW>(kbg + (int64_t)(key0 - kTile) * a.ksl, a.ksl, kTile, lds0 + (uint32_t)(((t + 1) & 1) * TILE * 2));
    f32x16 s[kTile / 32];
    float tm2 = -INFINITY;
    if (wave_busy) {
      qk_tile<kTile, false>(Ks, kofs, qf, s);
      const bool need_mask = nk < kTile || (a.causal && key0 + kTile - 1 > wave_min_pos) || !valid ||
                             qt * kTile + 32 * wr + 31 >= a.Lq;
      if (need_mask) {
        int lim = valid ? nk - 1 : -1;
        if (a.causal) lim = min(lim, row - key0);
        mask_tile<kTile / 32>(s, lim);
      }
      tm2 = tile_max<kTile / 32>(s) * a.c2;
      const bool vote = tm2 != -INFINITY && (m_run == -INFINITY || tm2 - m_run >= a.lnlam2);
      const unsigned long long bal = __ballot(vote);
      if (lane == 0) flags[w] = bal != 0ull;
    } else if (lane == 0) {
      flags[w] = 0;
    }
    __syncthreads();
    bool keep_any = false, keep = false;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      keep_any |= flags[x] != 0;
      if ((x >> 2) == hh) keep |= flags[x] != 0;
    }
    if (wr == 0 && lane == 0 && kmap) kmap[j] = keep ? 1 : 0;
    if (keep_any) issue_tile<kTile, NW>(vbg + (int64_t)key0 * a.vsl, a.vsl, nk, lds0 + (uint32_t)(2 * TILE * 2));
    if (keep) {
      ++nkept;
      if (wave_busy) {
        const float msub = softmax_rescale(tm2, m_run, l_run, o);
        softmax_probs<kTile / 32>(s, a.c2, msub, l_run);
      }
    }
    if (keep_any) {
      wait_tile_loads();                           // V of tile j (and K of tile j - 1)
      __syncthreads();
      if (keep && wave_busy) pv_tile<kTile>(Vs, vofs, s, o);
    }
  }

  if (wr == 0 && lane == 0 && a.kept) a.kept[((int64_t)b * Hq + h) * a.NQT + qt] = nkept;
  if (!valid) return;
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t oi = (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)row * a.osl;
  store_o_row(a.o_f32 ? (void*)(static_cast<float*>(a.o) + oi) : (void*)(static_cast<uint16_t*>(a.o) + oi),
              a.o_f32, o, inv, lane >> 5);
  if (lane < 32)
    a.lse[((int64_t)b * Hq + h) * a.Lq + row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

void launch_threshold(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const bsa_thresh_params& p,
                      const bsa_tensor& o, float* lse, int32_t* kept, uint8_t* keep_map, hipStream_t s) {
  ThrArgs a;
  a.q = static_cast<const uint16_t*>(q.data);
  a.k = static_cast<const uint16_t*>(k.data);
  a.v = static_cast<const uint16_t*>(v.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
  a.B = q.B; a.Hkv = k.H; a.G = q.H / k.H; a.L = k.L; a.Lq = q.L;
  a.NQT = (int)ceil_div(q.L, kTile);
  a.NKT = (int)ceil_div(k.L, kTile);
  a.causal = p.causal;
  a.c2 = p.scale * kLog2e;
  a.lnlam2 = p.lambda > 0.f ? (float)(std::log((double)p.lambda) * 1.4426950408889634) : -INFINITY;
  a.o = o.data; a.o_f32 = o.dtype == BSA_F32; a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
  a.lse = lse; a.kept = kept; a.keep_map = keep_map;
  if (a.G % 2 == 0) {
    dim3 grid(a.B * a.Hkv * a.NQT * (a.G / 2));
    hipLaunchKernelGGL(threshold_kernel<8>, grid, dim3(512), 0, s, a);
  } else {
    dim3 grid(a.B * a.Hkv * a.NQT * a.G);
    hipLaunchKernelGGL(threshold_kernel<4>, grid, dim3(256), 0, s, a);
  }
}

}  // namespace bsa
