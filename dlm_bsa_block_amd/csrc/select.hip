// Block selection: band temperatures, block logits, and per-query-block pick
// lists (top-k per GQA group with forced blocks, union over the block's rows).
//
// Scoring follows the mean-pooled key summary idea of the Prism page (sec. 1,
// and sec. 3 for the two RoPE bands with an energy temperature per band); the
// forced initial/newest blocks follow the NSA page's selection setting; the
// union over a query block follows the LoSA page (sec. 1-2).
//
// Three kernels:
//   tau_kernel     per (query head, batch): retained band energy of the pooled
//                  keys (and pooled queries) -> tau[b][h][band]
//   logits_kernel  LDS-tiled fp32 products z = scale * q.kmean (/ tau), written
//                  to workspace Z[b][g][row][head-in-group][band][block]
//   pick_kernel    per (query block, KV group, batch): per selection row, the
//                  per-head softmax over the candidates, the group score, a
//                  wavefront radix select of the k' best non-forced blocks
//                  (ties -> lower index), then an LDS bitmap union over rows
//                  and an ordered compaction to the sorted index list.
#include "common.cuh"
#include "internal.h"

namespace bsa {

// ------------------------------------------------------------- temperature ---
__device__ __forceinline__ void band_energy_ratio_terms(const float* __restrict__ mean, int64_t row_stride,
                                                        const float* __restrict__ energy, int nblk, int D, int layout,
                                                        float& nf, float& ns, float& df, float& ds) {
  // thread-strided partial sums in a fixed order
  nf = ns = df = ds = 0.f;
  const int tid = threadIdx.x;
  const int n = nblk * D;
  for (int i = tid; i < n; i += 256) {
    const int j = i / D, d = i - j * D;
    const float m = mean[(int64_t)j * row_stride + d];
    if (band_of_dim(d, D, layout) == 0) nf = fmaf(m, m, nf); else ns = fmaf(m, m, ns);
  }
  for (int j = tid; j < nblk; j += 256) { df += energy[2 * j]; ds += energy[2 * j + 1]; }
}

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_sum(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

__global__ __launch_bounds__(256) void tau_kernel(const float* __restrict__ k_mean, const float* __restrict__ k_energy,
                                                  int NB, const float* __restrict__ q_mean, int64_t qsb, int64_t qsh,
                                                  int64_t qsl, const float* __restrict__ q_energy, int NQB, int D,
                                                  int G, int layout, float* __restrict__ tau_ws,
                                                  float* __restrict__ tau_out) {
  __shared__ float sh[4];
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, Hkv = Hq / G, g = h / G;
  float nf, ns, df, ds;
  const int64_t kbase = ((int64_t)b * Hkv + g) * NB;
  band_energy_ratio_terms(k_mean + kbase * D, D, k_energy + kbase * 2, NB, D, layout, nf, ns, df, ds);
  float r[2];
  {
    const float a = block_sum256(nf, sh), c = block_sum256(ns, sh);
    const float e0 = block_sum256(df, sh), e1 = block_sum256(ds, sh);
    r[0] = e0 > 0.f ? a / e0 : 1.f;
    r[1] = e1 > 0.f ? c / e1 : 1.f;
  }
  if (q_mean != nullptr) {
    const int64_t qe = ((int64_t)b * Hq + h) * NQB;
    band_energy_ratio_terms(q_mean + b * qsb + h * qsh, qsl, q_energy + qe * 2, NQB, D, layout, nf, ns, df, ds);
    const float a = block_sum256(nf, sh), c = block_sum256(ns, sh);
    const float e0 = block_sum256(df, sh), e1 = block_sum256(ds, sh);
    r[0] *= e0 > 0.f ? a / e0 : 1.f;
    r[1] *= e1 > 0.f ? c / e1 : 1.f;
  }
  if (threadIdx.x < 2) {
    const float t = fmaxf(1e-6f, sqrtf(r[threadIdx.x]));
    tau_ws[((int64_t)b * Hq + h) * 2 + threadIdx.x] = t;
    if (tau_out) tau_out[((int64_t)b * Hq + h) * 2 + threadIdx.x] = t;
  }
}

// ------------------------------------------------------------------ logits ---
// Workgroup tile: TM query vectors (m = row * G + head-in-group) x TJ blocks.
// Thread (tx, ty) owns rows ty*RPT + r and blocks tx + TX*c.
template <int DT, int D, int TX, int TY, int RPT, int CPT, bool DUAL>
__global__ __launch_bounds__(256) void logits_kernel(const uint8_t* __restrict__ qdata, int64_t qsb, int64_t qsh,
                                                     int64_t qsl, const float* __restrict__ k_mean, int NB, int Rtot,
                                                     int G, int Hkv, float scale, const float* __restrict__ tau,
                                                     int layout, int causal, int q_block, int kv_block, int q_pos0,
                                                     int pooled, int Lq, float* __restrict__ Z) {
  constexpr int TM = TY * RPT, TJ = TX * CPT;
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int NBANDS = DUAL ? 2 : 1;
  __shared__ float Qs[TM][D + 1];
  __shared__ float Ks[TJ][D + 1];
  const int tid = threadIdx.x, tx = tid % TX, ty = tid / TX;
  const int j0 = blockIdx.x * TJ, m0 = blockIdx.y * TM;
  const int bg = blockIdx.z, b = bg / Hkv, g = bg - b * Hkv;
  const int M = Rtot * G;
  const int Hq = Hkv * G;

  if (causal) {
    // highest selection row of the tile -> its last visible block
    const int rmax = min(M - 1, m0 + TM - 1) / G;
    const int last_row = pooled ? min((rmax + 1) * q_block, Lq) - 1 : rmax;
    const int jmax = (q_pos0 + last_row) / kv_block;
    if (j0 > jmax) return;
  }

  // stage the query vectors (converted to f32) and the pooled keys
  for (int i = tid; i < TM * (D / 8); i += 256) {
    const int mm = i / (D / 8), d8 = (i - mm * (D / 8)) * 8;
    const int m = m0 + mm;
    float v[8];
    if (m < M) {
      const int row = m / G, hl = m - row * G;
      const uint8_t* p = qdata + ((int64_t)b * qsb + (int64_t)(g * G + hl) * qsh + (int64_t)row * qsl + d8) * ES;
      load8<DT>(p, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) Qs[mm][d8 + e] = v[e];
  }
  const float* kb = k_mean + ((int64_t)b * Hkv + g) * NB * D;
  for (int i = tid; i < TJ * (D / 4); i += 256) {
    const int jj = i / (D / 4), d4 = (i - jj * (D / 4)) * 4;
    const int j = j0 + jj;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < NB) v = *reinterpret_cast<const f32x4*>(kb + (int64_t)j * D + d4);
#pragma unroll
    for (int e = 0; e < 4; ++e) Ks[jj][d4 + e] = v[e];
  }
  __syncthreads();

  float acc[RPT][CPT][NBANDS];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int n = 0; n < NBANDS; ++n) acc[r][c][n] = 0.f;

#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    // a quarter of the dims always belongs to one band (either layout)
    const int bnd = DUAL ? ((layout == BSA_ROPE_HALF) ? (q4 & 1) : (q4 >> 1)) : 0;
#pragma unroll 8
    for (int d = q4 * (D / 4); d < (q4 + 1) * (D / 4); ++d) {
      float qv[RPT], kv[CPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) qv[r] = Qs[ty * RPT + r][d];
#pragma unroll
      for (int c = 0; c < CPT; ++c) kv[c] = Ks[tx + TX * c][d];
#pragma unroll
      for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          if (DUAL) {
            if (bnd == 0) acc[r][c][0] = fmaf(qv[r], kv[c], acc[r][c][0]);
            else acc[r][c][NBANDS - 1] = fmaf(qv[r], kv[c], acc[r][c][NBANDS - 1]);
          } else {
            acc[r][c][0] = fmaf(qv[r], kv[c], acc[r][c][0]);
          }
        }
    }
  }

#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int m = m0 + ty * RPT + r;
    if (m >= M) continue;
    const int row = m / G, hl = m - row * G;
    float inv_t[NBANDS];
#pragma unroll
    for (int n = 0; n < NBANDS; ++n)
      inv_t[n] = DUAL ? scale / tau[((int64_t)b * Hq + g * G + hl) * 2 + n] : scale;
    float* zr = Z + ((((int64_t)b * Hkv + g) * Rtot + row) * G + hl) * NBANDS * NB;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int j = j0 + tx + TX * c;
      if (j >= NB) continue;
#pragma unroll
      for (int n = 0; n < NBANDS; ++n) zr[(int64_t)n * NB + j] = acc[r][c][n] * inv_t[n];
    }
  }
}

// -------------------------------------------------------------------- pick ---
struct PickArgs {
  const float* Z;
  int NB, Rtot, G, Hkv, nbands;
  int q_block, kv_block, q_pos0, Lq, causal, pooled;
  int topk, topk_num, topk_den, n_first, n_last, cap;
  const uint8_t* row_mask;
  int32_t* idx;
  int32_t* cnt;
  int32_t* row_picks;
};

// Wavefront radix select on 32-bit keys (0 = not a candidate): finds the
// k-th largest key T and how many keys equal to T belong to the top k.
// Four 8-bit digit passes, most significant first, with a per-wave LDS
// histogram and a wave prefix scan over the digits in descending order.
template <typename KeyFn>
__device__ void wave_radix_select(KeyFn keyof, int n, int k, uint32_t* hist, uint32_t& T, int& need_eq) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = lane; i < 256; i += 64) hist[i] = 0u;
    wave_sync_lds();
    for (int j = lane; j < n; j += 64) {
      const uint32_t key = keyof(j);
      if (key != 0u && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    wave_sync_lds();
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; tot += c[i]; }
    uint32_t incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    uint32_t run = incl - tot;
    int found = -1;
    uint32_t above = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (found < 0 && run < (uint32_t)remaining && run + c[i] >= (uint32_t)remaining) {
        found = 255 - 4 * lane - i;
        above = run;
      }
      run += c[i];
    }
    const unsigned long long bal = __ballot(found >= 0);
    const int src = __ffsll((long long)bal) - 1;
    found = __shfl(found, src, 64);
    above = __shfl(above, src, 64);
    remaining -= (int)above;
    prefix |= (uint32_t)found << shift;
    pmask |= 0xFFu << shift;
    wave_sync_lds();
  }
  T = prefix;
  need_eq = remaining;
}

// Ordered compaction of a bitmap (nw <= 128 words) into ascending indices,
// padding out[total .. pad_to) with -1; returns the count.
__device__ int wave_compact(const uint32_t* bits, int nw, int32_t* out, int pad_to) {
  const int lane = threadIdx.x & 63;
  const uint32_t w0 = (2 * lane < nw) ? bits[2 * lane] : 0u;
  const uint32_t w1 = (2 * lane + 1 < nw) ? bits[2 * lane + 1] : 0u;
  const int c = __popc(w0) + __popc(w1);
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  int pos = incl - c;
  const int total = __shfl(incl, 63, 64);
  uint32_t wd = w0;
  for (int k = 0; k < 2; ++k) {
    const int base = (2 * lane + k) * 32;
    while (wd) {
      const int bit = __ffs(wd) - 1;
      out[pos++] = base + bit;
      wd &= wd - 1;
    }
    wd = w1;
  }
  for (int i = total + lane; i < pad_to; i += 64) out[i] = -1;
  return total;
}

constexpr int kPickMaxWords = 128;   // NB <= 4096

__device__ __forceinline__ size_t pick_wave_bytes(int NB) { return (size_t)NB * 4 + 256 * 4 + kPickMaxWords * 4; }

__global__ __launch_bounds__(256) void pick_kernel(PickArgs a) {
  extern __shared__ uint32_t smem[];
  const int NB = a.NB, NBW = (NB + 31) / 32;
  const int W = blockDim.x / 64, w = threadIdx.x / 64, lane = threadIdx.x & 63;
  uint32_t* ubits = smem;                                              // [128] union bitmap
  uint8_t* wbase = reinterpret_cast<uint8_t*>(smem + kPickMaxWords) + (size_t)w * pick_wave_bytes(NB);
  float* s = reinterpret_cast<float*>(wbase);                          // [NB] group scores
  uint32_t* hist = reinterpret_cast<uint32_t*>(s + NB);                // [256]
  uint32_t* rbits = hist + 256;                                        // [128] this row's picks

  const int qb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hkv = a.Hkv, G = a.G, NQB = gridDim.x;
  const int rows = a.pooled ? 1 : min(a.q_block, a.Lq - qb * a.q_block);
  // candidates [0, jmax], forced blocks, and the number of scored picks
  int jmax = NB - 1;
  if (a.causal) {
    const int last_row = min((qb + 1) * a.q_block, a.Lq) - 1;
    jmax = min(NB - 1, (a.q_pos0 + last_row) / a.kv_block);
  }
  const int nC = jmax + 1;
  const int nf_first = min(a.n_first, nC);
  const int last_lo = max(nf_first, nC - a.n_last);          // forced: j < nf_first or j >= last_lo
  const int n_forced = nf_first + (nC - last_lo);
  int kp = a.topk_num > 0 ? (int)(((int64_t)a.topk_num * nC + a.topk_den - 1) / a.topk_den) : a.topk;
  kp = max(0, min(kp, nC - n_forced));
  const int n_free = nC - n_forced;

  for (int i = threadIdx.x; i < kPickMaxWords; i += blockDim.x) ubits[i] = 0u;
  __syncthreads();

  for (int rl = w; rl < rows; rl += W) {
    const int row = a.pooled ? qb : qb * a.q_block + rl;
    int32_t* rp = a.row_picks ? a.row_picks + (((int64_t)b * Hkv + g) * a.Rtot + row) * a.cap : nullptr;
    if (!a.pooled && a.row_mask && a.row_mask[(int64_t)b * a.Lq + row] == 0) {
      if (rp) for (int i = lane; i < a.cap; i += 64) rp[i] = -1;
      continue;
    }
    for (int i = lane; i < kPickMaxWords; i += 64) rbits[i] = 0u;
    for (int j = lane; j < nC; j += 64) s[j] = 0.f;
    // group score: sum over heads (and bands) of softmax probabilities, fixed order
    const float wband = a.nbands == 2 ? 0.5f : 1.0f;
    for (int hl = 0; hl < G; ++hl) {
      for (int bd = 0; bd < a.nbands; ++bd) {
        const float* z = a.Z + (((((int64_t)b * Hkv + g) * a.Rtot + row) * G + hl) * a.nbands + bd) * NB;
        float mx = -INFINITY;
        for (int j = lane; j < nC; j += 64) mx = fmaxf(mx, z[j]);
        mx = wave_max(mx);
        float sm = 0.f;
        for (int j = lane; j < nC; j += 64) sm += expf(z[j] - mx);
        sm = wave_sum(sm);
        const float inv = wband / sm;
        for (int j = lane; j < nC; j += 64) s[j] = fmaf(expf(z[j] - mx), inv, s[j]);
      }
    }
    wave_sync_lds();
    auto keyof = [&](int j) -> uint32_t {
      const bool free_ = (j >= nf_first) && (j < last_lo);
      return free_ ? __float_as_uint(s[j]) + 1u : 0u;
    };
    uint32_t T = 0xFFFFFFFFu;
    int need_eq = 0;
    if (kp > 0 && kp < n_free) {
      wave_radix_select(keyof, nC, kp, hist, T, need_eq);
    } else if (kp > 0) {
      T = 1u;                       // take every non-forced candidate
      need_eq = 0x7FFFFFFF;
    }
    int taken = 0;
    for (int j0 = 0; j0 < nC; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t key = j < nC ? keyof(j) : 0u;
      const bool forced = j < nC && (j < nf_first || j >= last_lo);
      const bool gt = key != 0u && key > T;
      const bool eq = key != 0u && key == T;
      const unsigned long long m = __ballot(eq);
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      const bool take = forced || gt || (eq && taken + rank < need_eq);
      taken += __popcll(m);
      if (take) atomicOr(&rbits[j >> 5], 1u << (j & 31));
    }
    wave_sync_lds();
    for (int i = lane; i < NBW; i += 64) {
      const uint32_t v = rbits[i];
      if (v) atomicOr(&ubits[i], v);
    }
    if (rp) wave_compact(rbits, NBW, rp, a.cap);
    wave_sync_lds();
  }
  __syncthreads();
  if (w == 0) {
    const int64_t li = ((int64_t)b * Hkv + g) * NQB + qb;
    const int n = wave_compact(ubits, NBW, a.idx + li * a.cap, 0);
    if (lane == 0) a.cnt[li] = n;
  }
}

// ------------------------------------------------------------------- host ---
bool plan_select(const bsa_tensor& q, int NB, const bsa_select_params& p, SelectPlan& pl) {
  pl.B = q.B;
  pl.Hq = q.H;
  pl.D = q.D;
  pl.NB = NB;
  if (p.pooled_q) {
    pl.NQB = q.L;
    pl.Lq = p.q_len > 0 ? p.q_len : q.L * p.q_block;
    pl.R = 1;
  } else {
    pl.Lq = q.L;
    pl.NQB = (int)ceil_div(q.L, p.q_block);
    pl.R = p.q_block;
  }
  const int maxC = NB;
  int kp = p.topk_num > 0 ? (int)ceil_div((int64_t)p.topk_num * maxC, p.topk_den) : p.topk;
  pl.kp_max = kp;
  pl.cap = p.cap;
  return true;
}

static size_t pick_smem_bytes(int NB, int W) {
  return kPickMaxWords * 4 + (size_t)W * ((size_t)NB * 4 + 256 * 4 + kPickMaxWords * 4);
}

void launch_select(const bsa_tensor& q, const float* q_energy, const float* k_mean, const float* k_energy,
                   const bsa_select_params& p, const SelectPlan& pl, const uint8_t* row_mask, int32_t* idx,
                   int32_t* cnt, int32_t* row_picks, float* tau_out, void* ws, hipStream_t s) {
  const int G = pl.G, Hkv = pl.Hkv, NB = pl.NB;
  const int Rtot = p.pooled_q ? pl.NQB : pl.Lq;
  const int nb = p.dual_band ? 2 : 1;
  float* Z = static_cast<float*>(ws);
  float* tau = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.z_bytes);
  if (p.dual_band) {
    const float* qm = p.pooled_q ? static_cast<const float*>(q.data) : nullptr;
    hipLaunchKernelGGL(tau_kernel, dim3(pl.Hq, pl.B), dim3(256), 0, s, k_mean, k_energy, NB, qm, q.stride_b,
                       q.stride_h, q.stride_l, q_energy, pl.NQB, pl.D, G, p.layout, tau, tau_out);
  }
  const int M = Rtot * G;
  const uint8_t* qd = static_cast<const uint8_t*>(q.data);
#define BSA_LOGITS(DT, DD, TX, TY, RPT, CPT, DUAL)                                                        \
  do {                                                                                                    \
    dim3 grid((unsigned)ceil_div(NB, TX * CPT), (unsigned)ceil_div(M, TY * RPT), (unsigned)(pl.B * Hkv)); \
    hipLaunchKernelGGL((logits_kernel<DT, DD, TX, TY, RPT, CPT, DUAL>), grid, dim3(256), 0, s, qd,        \
                       q.stride_b, q.stride_h, q.stride_l, k_mean, NB, Rtot, G, Hkv, p.scale, tau, p.layout, \
                       p.causal, p.q_block, p.kv_block, p.q_pos0, p.pooled_q, pl.Lq, Z);                 \
  } while (0)
#define BSA_LOGITS_SHAPE(DT, DD, DUAL)                   \
  do {                                                   \
    if (M <= 8) BSA_LOGITS(DT, DD, 64, 4, 2, 1, DUAL);   \
    else BSA_LOGITS(DT, DD, 16, 16, 2, 4, DUAL);         \
  } while (0)
#define BSA_LOGITS_D(DT, DUAL)                                              \
  do {                                                                      \
    if (pl.D == 128) BSA_LOGITS_SHAPE(DT, 128, DUAL);                       \
    else BSA_LOGITS_SHAPE(DT, 64, DUAL);                                    \
  } while (0)
  if (q.dtype == BSA_BF16) {
    if (p.dual_band) BSA_LOGITS_D(BSA_BF16, true); else BSA_LOGITS_D(BSA_BF16, false);
  } else {
    if (p.dual_band) BSA_LOGITS_D(BSA_F32, true); else BSA_LOGITS_D(BSA_F32, false);
  }
#undef BSA_LOGITS_D
#undef BSA_LOGITS_SHAPE
#undef BSA_LOGITS

  PickArgs a;
  a.Z = Z;
  a.NB = NB;
  a.Rtot = Rtot;
  a.G = G;
  a.Hkv = Hkv;
  a.nbands = nb;
  a.q_block = p.q_block;
  a.kv_block = p.kv_block;
  a.q_pos0 = p.q_pos0;
  a.Lq = pl.Lq;
  a.causal = p.causal;
  a.pooled = p.pooled_q;
  a.topk = p.topk;
  a.topk_num = p.topk_num;
  a.topk_den = p.topk_den;
  a.n_first = p.n_first;
  a.n_last = p.n_last;
  a.cap = p.cap;
  a.row_mask = row_mask;
  a.idx = idx;
  a.cnt = cnt;
  a.row_picks = row_picks;
  const int W = p.pooled_q ? 1 : (pl.R >= 4 ? 4 : pl.R);
  const size_t smem = pick_smem_bytes(NB, W);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&pick_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL(pick_kernel, dim3(pl.NQB, Hkv, pl.B), dim3(64 * W), smem, s, a);
}

}  // namespace bsa
