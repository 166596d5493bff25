// Block selection: band temperatures, block logits, and per-query-block pick
// lists (top-k per GQA group with forced blocks, union over the block's rows).
//
// Scoring follows the mean-pooled key summary idea of the Prism page (sec. 1,
// and sec. 3 for the two RoPE bands with an energy temperature per band); the
// forced initial/newest blocks follow the NSA page's selection setting; the
// union over a query block follows the LoSA page (sec. 1-2).
//
// Kernels:
//   tau_partial_kernel  per (chunk of pooled vectors, head): band sums of the
//                       pooled vectors' squared norms and of the mean energies
//   tau_final_kernel    per (query head, batch): chunk sums in order ->
//                       tau[b][h][band]
//   logits_kernel       LDS-tiled fp32 products z = scale * q.kmean (/ tau),
//                       written to workspace Z[b][g][row][head-in-group][band][block]
//   pick_kernel         one workgroup per (selection row, KV group, batch):
//                       per-head (per-band) softmax over the candidates, group
//                       score; then one wave selects the k' best non-forced
//                       blocks (ties -> lower index; wave_select.h: a bitonic
//                       sort of the lanes' maxima bounds the k'-th key, the
//                       keys above the bound are ranked exactly).  With one
//                       selection row per query block the picks go straight
//                       into the sorted index list; otherwise every row
//                       writes its bitmap to the workspace
//   union_kernel        per (query block, KV group, batch): OR of the rows'
//                       bitmaps and an ordered compaction into the list
// No atomics are used: every list is a function of the inputs alone.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "locality.h"
#include "pick.h"
#include "wave_select.h"

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
  v = wave_sum_dpp(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// Partial band sums of one chunk of kTauChunk pooled vectors: for K (one
// workgroup per (chunk, KV head)) and, when queries are pooled, for Q (per
// (chunk, query head)).  part[b][id][chunk] = {sum |mean|^2 fast band, slow
// band, sum energy fast, slow}, id = KV head, or Hkv + query head.
__global__ __launch_bounds__(256) void tau_partial_kernel(const float* __restrict__ k_mean,
                                                          const float* __restrict__ k_energy, int NB,
                                                          const float* __restrict__ q_mean, int64_t qsb, int64_t qsh,
                                                          int64_t qsl, const float* __restrict__ q_energy, int NQB,
                                                          int D, int Hkv, int Hq, int layout, int nchunk,
                                                          float* __restrict__ part) {
  __shared__ float sh[4];
  const int c = blockIdx.x, id = blockIdx.y, b = blockIdx.z;
  const bool is_q = id >= Hkv;
  const int nblk = is_q ? NQB : NB;
  const int j0 = c * kTauChunk, j1 = min(nblk, j0 + kTauChunk);
  float nf = 0.f, ns = 0.f, df = 0.f, ds = 0.f;
  if (j0 < nblk) {
    const float* mean;
    const float* energy;
    int64_t rs;
    if (is_q) {
      const int h = id - Hkv;
      mean = q_mean + b * qsb + h * qsh + (int64_t)j0 * qsl;
      rs = qsl;
      energy = q_energy + (((int64_t)b * Hq + h) * NQB + j0) * 2;
    } else {
      mean = k_mean + (((int64_t)b * Hkv + id) * NB + j0) * D;
      rs = D;
      energy = k_energy + (((int64_t)b * Hkv + id) * NB + j0) * 2;
    }
    band_energy_ratio_terms(mean, rs, energy, j1 - j0, D, layout, nf, ns, df, ds);
  }
  const float a0 = block_sum256(nf, sh), a1 = block_sum256(ns, sh);
  const float e0 = block_sum256(df, sh), e1 = block_sum256(ds, sh);
  if (threadIdx.x == 0) {
    float* o = part + (((int64_t)b * (Hkv + Hq) + id) * nchunk + c) * 4;
    o[0] = a0; o[1] = a1; o[2] = e0; o[3] = e1;
  }
}

// Temperature per (query head, band) from the chunk sums, added in chunk
// order: tau = max(1e-6, sqrt(rho_K (* rho_Q))), rho = pooled / mean energy.
__global__ __launch_bounds__(64) void tau_final_kernel(const float* __restrict__ part, int Hkv, int G, int nchunk,
                                                       int with_q, float* __restrict__ tau_ws,
                                                       float* __restrict__ tau_out) {
  const int h = blockIdx.x, b = blockIdx.y, Hq = Hkv * G;
  if (threadIdx.x >= 2) return;
  const int band = threadIdx.x;
  auto ratio = [&](int id) {
    const float* p = part + ((int64_t)b * (Hkv + Hq) + id) * nchunk * 4;
    float num = 0.f, den = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      num += p[c * 4 + band];
      den += p[c * 4 + 2 + band];
    }
    return den > 0.f ? num / den : 1.f;
  };
  float r = ratio(h / G);
  if (with_q) r *= ratio(Hkv + h);
  const float t = fmaxf(1e-6f, sqrtf(r));
  tau_ws[((int64_t)b * Hq + h) * 2 + band] = t;
  if (tau_out) tau_out[((int64_t)b * Hq + h) * 2 + band] = t;
}

// -------------------------------------------------------------------- pick ---
// Sum of a value over the 256 threads, identical bits in every thread
// (fixed DPP order inside each wave, then the 4 wave totals in order).
__device__ __forceinline__ float block_sum(float v, float* red, int slot) {
  v = wave_sum_dpp(v);
  if ((threadIdx.x & 63) == 0) red[slot * 4 + (threadIdx.x >> 6)] = v;
  __syncthreads();
  return red[slot * 4] + red[slot * 4 + 1] + red[slot * 4 + 2] + red[slot * 4 + 3];
}
__device__ __forceinline__ float block_max(float v, float* red, int slot) {
  v = wave_max_dpp(v);
  if ((threadIdx.x & 63) == 0) red[slot * 4 + (threadIdx.x >> 6)] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[slot * 4], red[slot * 4 + 1]), fmaxf(red[slot * 4 + 2], red[slot * 4 + 3]));
}
// The first n of N maxima (or sums) over the 256 threads behind a single
// barrier, in slots slot0 .. slot0 + N - 1; same fixed order as the one-value
// forms.
template <int N>
__device__ __forceinline__ void block_max_n(float (&v)[N], int n, float* red, int slot0) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) v[i] = wave_max_dpp(v[i]);                   // n is uniform: unused values skip the reduction
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red[(slot0 + i) * 4 + (threadIdx.x >> 6)] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float* r = red + (slot0 + i) * 4;
    v[i] = fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
  }
}
// Sum over the 256 threads in the order shared with the per-wave pick of the
// denoising step: for each lane l the partials of threads l, 64 + l, 128 + l
// and 192 + l are added in that order, then the 64 lane sums go through the
// DPP network; every thread gets the same bits.  red: N * 256 floats.
template <int N>
__device__ __forceinline__ void block_sum_lanes_n(float (&v)[N], float* red) {
  const int t = threadIdx.x, l = t & 63;
#pragma unroll
  for (int i = 0; i < N; ++i) red[i * 256 + t] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = ((red[i * 256 + l] + red[i * 256 + 64 + l]) + red[i * 256 + 128 + l]) + red[i * 256 + 192 + l];
  wave_sum_dpp_n<N>(v);
}

// Ordered compaction of a bitmap (nw <= 128 words) into ascending indices,
// padding out[total .. pad_to) with -1; returns the count.  One wavefront.
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

// One workgroup per (selection row, KV group, batch).  Thread t owns the
// candidates j = t + 256*u.  Per (head, band) channel: block-wide max, sum of
// exp2 (logits are in log2 units; summed in the order block_sum_lanes_n
// fixes), then the group score s[j] = sum over channels of w * exp2(z - M) / S
// in a fixed channel order, kept in registers.
// The scores go to LDS as order-preserving keys and one wavefront takes the k'
// best free candidates (ties -> lower index; wave_topk) and adds the forced
// blocks.  Blocks with one selection row write their sorted list directly;
// otherwise the row's bitmap goes to the workspace for the union kernel.
template <int U>
__global__ __launch_bounds__(kPickThreads) void pick_kernel(PickArgs a) {
  constexpr int KPL = 4 * U;                          // keys per lane of the selecting wave
  __shared__ uint32_t keys_sh[kPickThreads * U];
  __shared__ float red[2 * kPickChanBatch * 4];
  __shared__ float red2[kPickChanBatch * kPickThreads];
  __shared__ __attribute__((aligned(16))) uint32_t cand_sh[64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const RowPlan rp = row_plan(a, row);
  const int NBW = (a.NB + 31) / 32, nC = rp.nC, NBp = a.NBp;
  const int nchan = a.G * a.nbands;
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + rp.qb;
  const float* zrow = a.Z + (((int64_t)b * a.Hkv + g) * a.Rtot + row) * (int64_t)nchan * NBp;
  constexpr int CC = kPickRegs / U > kPickChanBatch ? kPickChanBatch : (kPickRegs / U > 0 ? kPickRegs / U : 1);
  // logits of a batch of channels: every load is requested (from a clamped, valid slot) before
  // any is used, and slots past the channels or candidates become -inf afterwards
  auto load_z = [&](int c0, float (&z)[CC][U]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < CC; ++cc)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = tid + kPickThreads * u;
        z[cc][u] = zrow[(int64_t)min(c0 + cc, nchan - 1) * NBp + min(j, nC - 1)];
      }
#pragma unroll
    for (int cc = 0; cc < CC; ++cc)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (!(c0 + cc < nchan && tid + kPickThreads * u < nC)) z[cc][u] = -INFINITY;
  };
  float z0[CC][U];
  load_z(0, z0);                                      // requested before the row mask is looked at
  const bool active = a.pooled || !a.row_mask || a.row_mask[(int64_t)b * a.Lq + row] != 0;
  if (active) {
    const float wband = a.nbands == 2 ? 0.5f : 1.0f;
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) s[u] = 0.f;
    for (int c0 = 0; c0 < nchan; c0 += CC) {
      float z[CC][U];
      if (c0 == 0) {
#pragma unroll
        for (int cc = 0; cc < CC; ++cc)
#pragma unroll
          for (int u = 0; u < U; ++u) z[cc][u] = z0[cc][u];
      } else {
        load_z(c0, z);
      }
      // all channels of the batch share the two barriers of their max and sum
      float mx[CC], sm[CC];
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        mx[cc] = z[cc][0];
#pragma unroll
        for (int u = 1; u < U; ++u) mx[cc] = fmaxf(mx[cc], z[cc][u]);
      }
      const int nb = min(CC, nchan - c0);             // channels in this batch
      block_max_n<CC>(mx, nb, red, 0);
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        sm[cc] = 0.f;
        if (c0 + cc >= nchan) continue;                 // uniform over the workgroup
#pragma unroll
        for (int u = 0; u < U; ++u) {
          z[cc][u] = fast_exp2(z[cc][u] - mx[cc]);      // -inf (not a candidate) -> 0
          sm[cc] += z[cc][u];
        }
      }
      block_sum_lanes_n<CC>(sm, red2);
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        if (c0 + cc >= nchan) continue;
        const float inv = wband / sm[cc];
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = fmaf(z[cc][u], inv, s[u]);
      }
      __syncthreads();                                  // red[] and red2[] are reused by the next batch
    }
    // keys: free candidates only; scores are >= 0, so float bits order like values
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + kPickThreads * u;
      keys_sh[j] = (j < nC && j >= rp.nf_first && j < rp.last_lo) ? __float_as_uint(s[u]) + 1u : 0u;
    }
  }
  __syncthreads();
  if (w != 0) return;
  uint64_t flags = 0;
  if (active) {
    uint32_t k[KPL];                                  // lane l holds blocks KPL l .. KPL l + KPL - 1
#pragma unroll
    for (int i = 0; i < KPL; ++i) k[i] = keys_sh[KPL * lane + i];
    flags = wave_topk<KPL>(k, rp.kp, rp.n_free, cand_sh);
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int j = KPL * lane + i;
      if (j < nC && (j < rp.nf_first || j >= rp.last_lo)) flags |= 1ull << i;    // forced blocks
    }
  }
  if (a.row_picks)
    wave_flags_to_list<KPL>(flags, a.row_picks + (((int64_t)b * a.Hkv + g) * a.Rtot + row) * a.cap, a.cap);
  if (!a.multi_row) {
    const int n = wave_flags_to_list<KPL>(flags, a.idx + li * a.cap, 0);
    if (lane == 0) a.cnt[li] = n;
  } else {
    wave_flags_to_bits<KPL>(flags, a.row_bits + (((int64_t)b * a.Hkv + g) * a.Rtot + row) * kPickMaxWords, NBW);
  }
}

// Union of the rows' picks of each query block (blocks with several rows):
// OR of the row bitmaps, then an ordered compaction.  One wavefront per block.
__global__ __launch_bounds__(64) void union_kernel(PickArgs a) {
  __shared__ uint32_t bits[kPickMaxWords];
  const int qb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int NBW = (a.NB + 31) / 32;
  const int rows = min(a.q_block, a.Lq - qb * a.q_block);
  const uint32_t* first = a.row_bits + (((int64_t)b * a.Hkv + g) * a.Rtot + (int64_t)qb * a.q_block) * kPickMaxWords;
  for (int i = lane; i < NBW; i += 64) {
    uint32_t u = 0u;
    for (int r0 = 0; r0 < rows; r0 += 32) {
      // rows past the block's end re-read its last row (OR is idempotent): no load under a branch
      uint32_t v[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = first[(int64_t)min(r0 + k, rows - 1) * kPickMaxWords + i];
#pragma unroll
      for (int k = 0; k < 32; ++k) u |= v[k];
    }
    bits[i] = u;
  }
  wave_sync_lds();
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  const int n = wave_compact(bits, NBW, a.idx + li * a.cap, 0);
  if (lane == 0) a.cnt[li] = n;
}

// ------------------------------------------------------------------ logits ---
// Workgroup tile: TM query vectors (m = row * G + head-in-group) x TJ blocks.
// Thread (tx, ty) owns rows ty*RPT + r and blocks tx + TX*c.
// Logits are written in log2 units (scale includes log2(e)), so the pick stage
// can use exp2.
template <int DT, int D, int TX, int TY, int RPT, int CPT, bool DUAL>
__global__ __launch_bounds__(256) void logits_kernel(const uint8_t* __restrict__ qdata, int64_t qsb, int64_t qsh,
                                                     int64_t qsl, const float* __restrict__ k_mean, int NB, int Rtot,
                                                     int G, int Hkv, float scale, const float* __restrict__ tau,
                                                     int layout, int causal, int q_block, int kv_block, int q_pos0,
                                                     int pooled, int Lq, float* __restrict__ Z, RefreshArgs ra,
                                                     ActiveRowsArgs act) {
  if (act.a != nullptr && (int)blockIdx.z >= act.z0) {
    // the denoising step's active-row test rides in this launch: extra z-slices, one row per workgroup
    __shared__ float sh4[4];
    const int k = blockIdx.z - act.z0, b = k / act.slices;
    const int r = (k - b * act.slices) * (gridDim.x * gridDim.y) + blockIdx.y * gridDim.x + blockIdx.x;
    if (r < act.R) active_row_job<DT>(act, r, b, sh4);
    return;
  }
  constexpr int TM = TY * RPT, TJ = TX * CPT;
  const int NBp = (NB + 3) & ~3;          // row stride of Z, a multiple of 4 floats
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int NBANDS = DUAL ? 2 : 1;
  // rows padded to D + 4 floats: 16-byte reads of 4 dims, and the 16 lanes of a row group hit
  // distinct banks (row stride 132 words = 4 banks apart)
  __shared__ __attribute__((aligned(16))) float Qs[TM][D + 4];
  __shared__ __attribute__((aligned(16))) float Ks[TJ][D + 4];
  const int tid = threadIdx.x, tx = tid % TX, ty = tid / TX;
  const int j0 = blockIdx.x * TJ, m0 = blockIdx.y * TM;
  const int bg = blockIdx.z, b = bg / Hkv, g = bg - b * Hkv;
  const int M = Rtot * G;
  const int Hq = Hkv * G;

  if (causal) {
    // highest selection row of the tile -> its last visible block
    // (the candidates of a raw row are those of its whole query block, as in the pick)
    const int rmax = min(M - 1, m0 + TM - 1) / G;
    const int qbmax = pooled ? rmax : rmax / q_block;
    const int last_row = min((qbmax + 1) * q_block, Lq) - 1;
    const int jmax = (q_pos0 + last_row) / kv_block;
    if (j0 > jmax) return;
  }

  // stage the query vectors (converted to f32) and the pooled keys.  Every load of both is
  // requested before the first LDS store, from clamped (valid) addresses, and out-of-range
  // entries are zeroed afterwards: a load under a branch would make each wait for the last.
  const float* kb = k_mean + ((int64_t)b * Hkv + g) * NB * D;
  // the block being refreshed (the newest, whose tokens change every decode
  // step) is pooled here from K instead of read back, and written out
  const int jr = ra.block - j0;
  const bool refresh = ra.block >= 0 && jr >= 0 && jr < TJ;     // uniform over the workgroup
  constexpr int QN = TM * (D / 8), KN = TJ * (D / 4);
  constexpr int QIT = (QN + 255) / 256, KIT = (KN + 255) / 256;
  float qv[QIT][8];
  f32x4 kv[KIT];
#pragma unroll
  for (int u = 0; u < QIT; ++u) {
    const int i = min(tid + 256 * u, QN - 1);
    const int mm = i / (D / 8), d8 = (i - mm * (D / 8)) * 8;
    const int m = min(m0 + mm, M - 1);
    const int row = m / G, hl = m - row * G;
    load8<DT>(qdata + ((int64_t)b * qsb + (int64_t)(g * G + hl) * qsh + (int64_t)row * qsl + d8) * ES, qv[u]);
  }
#pragma unroll
  for (int u = 0; u < KIT; ++u) {
    const int i = min(tid + 256 * u, KN - 1);
    const int jj = i / (D / 4), d4 = (i - jj * (D / 4)) * 4;
    kv[u] = *reinterpret_cast<const f32x4*>(kb + (int64_t)min(j0 + jj, NB - 1) * D + d4);
  }
#pragma unroll
  for (int u = 0; u < QIT; ++u) {
    const int i = tid + 256 * u;
    if (i < QN) {
      const int mm = i / (D / 8), d8 = (i - mm * (D / 8)) * 8;
      const bool in = m0 + mm < M;
      *reinterpret_cast<f32x4*>(&Qs[mm][d8]) =
          in ? f32x4{qv[u][0], qv[u][1], qv[u][2], qv[u][3]} : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&Qs[mm][d8 + 4]) =
          in ? f32x4{qv[u][4], qv[u][5], qv[u][6], qv[u][7]} : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int u = 0; u < KIT; ++u) {
    const int i = tid + 256 * u;
    if (i < KN) {
      const int jj = i / (D / 4), d4 = (i - jj * (D / 4)) * 4;
      const bool in = j0 + jj < NB && !(refresh && jj == jr);
      *reinterpret_cast<f32x4*>(&Ks[jj][d4]) = in ? kv[u] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (refresh) {
    // one pass of 16 lanes x 8 dims per row, 16 rows per pass, fixed-order sums (as the summaries kernel)
    constexpr int LPR = D / 8, RPP = 256 / LPR;
    __shared__ float red[RPP][D + 4];
    __shared__ float ered[4][2];
    const int c = tid % LPR, rg = tid / LPR;
    const int t0 = ra.block * kv_block, n = min(kv_block, ra.L - t0);
    const uint8_t* kp = ra.k + ((int64_t)b * ra.ksb + (int64_t)g * ra.ksh + (int64_t)t0 * ra.ksl) * ES + c * 8 * ES;
    float sum[8], e2 = 0.f;
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) sum[q8] = 0.f;
    for (int r0 = 0; r0 < n; r0 += 4 * RPP) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<DT>(kp + (int64_t)min(r0 + u * RPP + rg, n - 1) * ra.ksl * ES, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = r0 + u * RPP + rg < n;
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) v[u][q8] = in ? v[u][q8] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) { sum[q8] += v[u][q8]; e2 = fmaf(v[u][q8], v[u][q8], e2); }
    }
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) red[rg][c * 8 + q8] = sum[q8];
    const int band = band_of_dim(c * 8, D, layout);
    float ef = band == 0 ? e2 : 0.f, es = band == 0 ? 0.f : e2;
    ef = wave_sum(ef);
    es = wave_sum(es);
    if ((tid & 63) == 0) { ered[tid >> 6][0] = ef; ered[tid >> 6][1] = es; }
    __syncthreads();
    const float inv = 1.0f / (float)n;
    const int64_t row = ((int64_t)b * Hkv + g) * NB + ra.block;
    for (int d = tid; d < D; d += 256) {
      float t = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) t += red[rr][d];
      t *= inv;
      Ks[jr][d] = t;
      if (blockIdx.y == 0) ra.mean[row * D + d] = t;
    }
    if (ra.energy && blockIdx.y == 0 && tid < 2) ra.energy[row * 2 + tid] = (ered[0][tid] + ered[1][tid] + ered[2][tid] + ered[3][tid]) * inv;
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
    // four dims per LDS read; the products are still accumulated one dim at a time, in order
#pragma unroll 2
    for (int d4 = q4 * (D / 4); d4 < (q4 + 1) * (D / 4); d4 += 4) {
      f32x4 qv[RPT], kv[CPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) qv[r] = *reinterpret_cast<const f32x4*>(&Qs[ty * RPT + r][d4]);
#pragma unroll
      for (int c = 0; c < CPT; ++c) kv[c] = *reinterpret_cast<const f32x4*>(&Ks[tx + TX * c][d4]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            if (DUAL) {
              if (bnd == 0) acc[r][c][0] = fmaf(qv[r][e], kv[c][e], acc[r][c][0]);
              else acc[r][c][NBANDS - 1] = fmaf(qv[r][e], kv[c][e], acc[r][c][NBANDS - 1]);
            } else {
              acc[r][c][0] = fmaf(qv[r][e], kv[c][e], acc[r][c][0]);
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
    float* zr = Z + ((((int64_t)b * Hkv + g) * Rtot + row) * G + hl) * NBANDS * NBp;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int j = j0 + tx + TX * c;
      if (j >= NB) continue;
#pragma unroll
      for (int n = 0; n < NBANDS; ++n) zr[(int64_t)n * NBp + j] = acc[r][c][n] * inv_t[n];
    }
  }
}

// Block logits on the matrix cores (raw bf16 query rows, D = 128, one band):
// Z = Q . Kmean^T per 32 x 32 tile with v_mfma_f32_32x32x16_bf16.  The query
// rows are bf16 already; each f32 summary x is split exactly into three bf16
// parts by truncation: hi = the top 8 significand bits of x, mid = the top 8 of
// x - hi, lo = x - hi - mid (at most 8 bits left; both differences are exact
// in fp32).  Every product is then exact and only the fp32 accumulation
// rounds, as in the vector form.  One workgroup = 4 waves over 128 query
// vectors x 32 blocks, each wave one 32 x 32 tile: the waves share the blocks'
// summaries (read from memory once per workgroup, the other waves hit the
// cache) and each summary is read by one workgroup only.  The operands go
// straight from memory into registers (every load requested before the first
// product), and no LDS is used.
__global__ __launch_bounds__(256) void logits_mfma_kernel(const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh,
                                                          int64_t qsl, const float* __restrict__ k_mean, int NB,
                                                          int Rtot, int G, int Hkv, float scale, int causal,
                                                          int q_block, int kv_block, int q_pos0, int Lq,
                                                          float* __restrict__ Z, ActiveRowsArgs act) {
  if (act.a != nullptr && (int)blockIdx.z >= act.z0) {
    __shared__ float sh4[4];
    const int k = blockIdx.z - act.z0, b = k / act.slices;
    const int r = (k - b * act.slices) * (gridDim.x * gridDim.y) + blockIdx.y * gridDim.x + blockIdx.x;
    if (r < act.R) active_row_job<BSA_BF16>(act, r, b, sh4);
    return;
  }
  constexpr int D = 128;
  const int NBp = (NB + 3) & ~3;
  const int M = Rtot * G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c32 = lane & 31, hi = lane >> 5;
  const int m0 = blockIdx.y * 128 + w * 32, j0 = blockIdx.x * 32;
  if (m0 >= M) return;                              // uniform over the wave; no barrier follows
  const int bg = blockIdx.z, b = bg / Hkv, g = bg - b * Hkv;
  if (causal) {
    // the tile's last row sees blocks up to jmax (the candidates of a raw row are its query block's)
    const int rmax = min(M - 1, m0 + 31) / G;
    const int last_row = min((rmax / q_block + 1) * q_block, Lq) - 1;
    if (j0 > (q_pos0 + last_row) / kv_block) return;   // uniform over the wave
  }
  // operands: query vector m0 + c32 (row m / G, head g G + m % G) and block j0 + c32, dims 16 t + 8 hi ..
  const int m = min(m0 + c32, M - 1), row = m / G, hl = m - row * G;
  const uint16_t* qp = q + (int64_t)b * qsb + (int64_t)(g * G + hl) * qsh + (int64_t)row * qsl + 8 * hi;
  const float* kp = k_mean + (((int64_t)b * Hkv + g) * NB + min(j0 + c32, NB - 1)) * D + 8 * hi;
  bf16x8 qa[8];
  f32x4 kv[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) qa[t] = *reinterpret_cast<const bf16x8*>(qp + 16 * t);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    kv[t][0] = *reinterpret_cast<const f32x4*>(kp + 16 * t);
    kv[t][1] = *reinterpret_cast<const f32x4*>(kp + 16 * t + 4);
  }
  // every load lands before the first product (left to itself the compiler issues the later k-steps'
  // loads between the products, each then a round trip of its own)
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    asm volatile("" : "+v"(qa[t]));
    asm volatile("" : "+v"(kv[t][0]), "+v"(kv[t][1]));
  }
  f32x16 acc_hi = f32x16{}, acc_lo = f32x16{};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t xb[8], r1b[8], r2b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = kv[t][e >> 2][e & 3];
      xb[e] = __float_as_uint(x);
      const float r1 = x - __uint_as_float(xb[e] & 0xFFFF0000u);
      r1b[e] = __float_as_uint(r1);
      r2b[e] = __float_as_uint(r1 - __uint_as_float(r1b[e] & 0xFFFF0000u));
    }
    // bf16 pairs: the upper halves of two words (the truncations; r2 has no lower half)
    u32x4 ph, pm, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ph[e] = __builtin_amdgcn_perm(xb[2 * e + 1], xb[2 * e], 0x07060302u);
      pm[e] = __builtin_amdgcn_perm(r1b[2 * e + 1], r1b[2 * e], 0x07060302u);
      pl[e] = __builtin_amdgcn_perm(r2b[2 * e + 1], r2b[2 * e], 0x07060302u);
    }
    acc_hi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], __builtin_bit_cast(bf16x8, ph), acc_hi, 0, 0, 0);
    acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], __builtin_bit_cast(bf16x8, pm), acc_lo, 0, 0, 0);
    acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], __builtin_bit_cast(bf16x8, pl), acc_lo, 0, 0, 0);
  }
  // lane: block j0 + c32; element i: query vector m0 + 8 (i / 4) + 4 hi + i % 4
  const int j = j0 + c32;
  if (j >= NB) return;
  float* zb = Z + (((int64_t)b * Hkv + g) * Rtot * G) * NBp + j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mm = m0 + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (mm < M) zb[(int64_t)mm * NBp] = (acc_hi[i] + acc_lo[i]) * scale;
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


PickArgs make_pick_args(const bsa_select_params& p, const SelectPlan& pl, void* ws, const uint8_t* row_mask,
                        int32_t* idx, int32_t* cnt, int32_t* row_picks) {
  PickArgs a;
  a.Z = static_cast<const float*>(ws);
  a.NB = pl.NB;
  a.NBp = (pl.NB + 3) & ~3;
  a.Rtot = p.pooled_q ? pl.NQB : pl.Lq;
  a.G = pl.G;
  a.Hkv = pl.Hkv;
  a.nbands = p.dual_band ? 2 : 1;
  a.NQB = pl.NQB;
  a.q_block = p.q_block;
  a.kv_block = p.kv_block;
  a.q_pos0 = p.q_pos0;
  a.Lq = pl.Lq;
  a.causal = p.causal;
  a.pooled = p.pooled_q;
  a.multi_row = (!p.pooled_q && std::min(p.q_block, pl.Lq) > 1) ? 1 : 0;
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
  a.row_bits = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + pl.z_bytes + pl.tau_bytes);
  return a;
}

// The block logits (after the band temperatures when dual-band), with the
// optional summary refresh and the optional active-row jobs in the same launch.
static void launch_logits(const bsa_tensor& q, const float* k_mean, const bsa_select_params& p, const SelectPlan& pl,
                          void* ws, hipStream_t s, const RefreshArgs& ra, ActiveRowsArgs act) {
  const int G = pl.G, Hkv = pl.Hkv, NB = pl.NB;
  const int Rtot = p.pooled_q ? pl.NQB : pl.Lq;
  float* Z = static_cast<float*>(ws);
  const float* tau = reinterpret_cast<const float*>(static_cast<uint8_t*>(ws) + pl.z_bytes);
  const int M = Rtot * G;
  const uint8_t* qd = static_cast<const uint8_t*>(q.data);
  const float scale2 = p.scale * kLog2e;
#define BSA_LOGITS(DT, DD, TX, TY, RPT, CPT, DUAL)                                                        \
  do {                                                                                                    \
    dim3 grid((unsigned)ceil_div(NB, TX * CPT), (unsigned)ceil_div(M, TY * RPT), (unsigned)(pl.B * Hkv)); \
    if (act.a) {                                                                                          \
      act.z0 = (int)grid.z;                                                                               \
      act.slices = (int)ceil_div(act.R, (int64_t)grid.x * grid.y);                                        \
      grid.z += (unsigned)(pl.B * act.slices);                                                            \
    }                                                                                                     \
    hipLaunchKernelGGL((logits_kernel<DT, DD, TX, TY, RPT, CPT, DUAL>), grid, dim3(256), 0, s, qd,        \
                       q.stride_b, q.stride_h, q.stride_l, k_mean, NB, Rtot, G, Hkv, scale2, tau, p.layout, \
                       p.causal, p.q_block, p.kv_block, p.q_pos0, p.pooled_q, pl.Lq, Z, ra, act);        \
  } while (0)
#define BSA_LOGITS_SHAPE(DT, DD, DUAL)                                   \
  do {                                                                   \
    if (M <= 8) BSA_LOGITS(DT, DD, 32, 8, 1, 1, DUAL);                   \
    else BSA_LOGITS(DT, DD, 16, 16, 2, 4, DUAL);                         \
  } while (0)
  if (M > 8 && q.dtype == BSA_BF16 && pl.D == 128 && !p.dual_band && !p.pooled_q && ra.block < 0) {
    // raw bf16 rows in tiles of 32: the matrix cores (one band, no refresh)
    dim3 grid((unsigned)ceil_div(NB, 32), (unsigned)ceil_div(M, 128), (unsigned)(pl.B * Hkv));
    if (act.a) {
      act.z0 = (int)grid.z;
      act.slices = (int)ceil_div(act.R, (int64_t)grid.x * grid.y);
      grid.z += (unsigned)(pl.B * act.slices);
    }
    hipLaunchKernelGGL(logits_mfma_kernel, grid, dim3(256), 0, s, reinterpret_cast<const uint16_t*>(qd),
                       q.stride_b, q.stride_h, q.stride_l, k_mean, NB, Rtot, G, Hkv, scale2, p.causal, p.q_block,
                       p.kv_block, p.q_pos0, pl.Lq, Z, act);
    return;
  }
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
}

void launch_select_logits(const bsa_tensor& q, const float* k_mean, const bsa_select_params& p,
                          const SelectPlan& pl, void* ws, hipStream_t s, const ActiveRowsArgs& act) {
  launch_logits(q, k_mean, p, pl, ws, s, RefreshArgs(), act);
}

void launch_select(const bsa_tensor& q, const float* q_energy, const float* k_mean, const float* k_energy,
                   const bsa_select_params& p, const SelectPlan& pl, const uint8_t* row_mask, int32_t* idx,
                   int32_t* cnt, int32_t* row_picks, float* tau_out, void* ws, hipStream_t s, const RefreshArgs& ra) {
  const int Hkv = pl.Hkv, NB = pl.NB;
  float* tau = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.z_bytes);
  if (p.dual_band) {
    const float* qm = p.pooled_q ? static_cast<const float*>(q.data) : nullptr;
    const int nchunk = tau_chunks(NB, p.pooled_q ? pl.NQB : 0);
    float* part = tau + align256((size_t)pl.B * pl.Hq * 2 * 4) / 4;
    const int ids = Hkv + (qm ? pl.Hq : 0);
    hipLaunchKernelGGL(tau_partial_kernel, dim3(nchunk, ids, pl.B), dim3(256), 0, s, k_mean, k_energy, NB, qm,
                       q.stride_b, q.stride_h, q.stride_l, q_energy, pl.NQB, pl.D, Hkv, pl.Hq, p.layout, nchunk,
                       part);
    hipLaunchKernelGGL(tau_final_kernel, dim3(pl.Hq, pl.B), dim3(64), 0, s, part, Hkv, pl.G, nchunk, qm ? 1 : 0, tau,
                       tau_out);
  }
  launch_logits(q, k_mean, p, pl, ws, s, ra, ActiveRowsArgs());
  const PickArgs a = make_pick_args(p, pl, ws, row_mask, idx, cnt, row_picks);
  const int Rtot = a.Rtot;
  const int U = (int)ceil_div(a.NBp, kPickThreads);
  dim3 pgrid(Rtot, Hkv, pl.B);
  if (U <= 1) hipLaunchKernelGGL(pick_kernel<1>, pgrid, dim3(kPickThreads), 0, s, a);
  else if (U <= 2) hipLaunchKernelGGL(pick_kernel<2>, pgrid, dim3(kPickThreads), 0, s, a);
  else if (U <= 4) hipLaunchKernelGGL(pick_kernel<4>, pgrid, dim3(kPickThreads), 0, s, a);
  else if (U <= 8) hipLaunchKernelGGL(pick_kernel<8>, pgrid, dim3(kPickThreads), 0, s, a);
  else hipLaunchKernelGGL(pick_kernel<16>, pgrid, dim3(kPickThreads), 0, s, a);
  if (a.multi_row)
    hipLaunchKernelGGL(union_kernel, dim3(pl.NQB, Hkv, pl.B), dim3(64), 0, s, a);
}

}  // namespace bsa
