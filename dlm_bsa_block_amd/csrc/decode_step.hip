// A decode step of selected-block attention in two launches.
//
//   dstep_logits_kernel   block logits of every decode row against the pooled
//                         key summaries (Prism sec. 1: a block is scored by the
//                         mean of its keys), with the newest block's summary
//                         pooled from K first when asked (its tokens change
//                         every step), plus each wavefront's softmax partials
//                         (max and sum of exp2 over its 8 blocks) per head
//   dstep_attend_kernel   per (slice of the list, row, KV group): the group
//                         scores s[j] = sum over the group's heads of
//                         softmax_h(z)[j] from the logits and the merged
//                         partials, the k' best plus the forced blocks (NSA
//                         structure section: block 0 and the newest ones) --
//                         computed identically by every workgroup of the
//                         group, so no launch sits between selection and
//                         attention -- then the workgroup's slice of the
//                         list's tokens, G query heads sharing each K/V load
//                         (NSA implementation section).  The slice's partial
//                         (m, l, o) is published with device-scope stores and
//                         counted; the workgroup that counts last merges all
//                         slices in order and writes O and LSE.
//
// Measured here: a kernel boundary costs about 4.5 us (the end-of-kernel cache
// write-back plus the next dispatch), a device-scope release fence about
// 10 us (it writes back the whole L2), a device-scope atomic or load 1-2 us.
// The logits need every summary of the group, hence the one boundary; the
// merge of the slices goes through device-scope stores and a counter, which
// need no fence.
//
// The lists, outputs and LSE are those of bsa_select_blocks_refresh followed
// by bsa_sparse_attention_fwd on the same arguments, up to fp32 rounding of the
// scores (the normalisers are summed in another order).
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "split.h"
#include "split_merge.h"
#include "dec_chunk.h"
#include "wave_select.h"

namespace bsa {

struct DStepArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl;
  float* k_mean;                  // [B][Hkv][NB][D]
  float* k_energy;                // [B][Hkv][NB][2] or null
  int refresh;                    // block pooled from K in this step, or -1
  int B, Hkv, Lq, L, NB, NBp, kv_block, q_pos0, causal, layout;
  int topk, topk_num, topk_den, n_first, n_last, cap;
  float c2;                       // scale * log2(e)
  float* Z;                       // [B][Hkv][Lq][G][NBp] logits (log2 units)
  float* stats;                   // [B][Hkv][Lq][G][P][2] per-wavefront (max, sum of exp2)
  int P;                          // wavefronts of the logits launch per row: 4 * ceil(NB / 32)
  int32_t* idx;
  int32_t* cnt;
  float* part_o;                  // [B][Hkv][Lq][items][G][D]
  float* part_ml;                 // [B][Hkv][Lq][items][G][2]
  uint32_t* arrivals;             // [B][Hkv][Lq] x 32 words: slices finished (zeroed by the logits launch)
  int items, tok_per_item;
  void* o;                        // [B][Hq][Lq][D], bf16 or f32
  int o_f32;
  int64_t osb, osh, osl;
  float* lse;                     // [B][Hq][Lq]
};

// ------------------------------------------------------------------ logits ---
// Workgroup = 4 waves x 8 blocks; 8 lanes per block, D / 8 dims per lane.  The
// workgroup that owns the newest block pools it from K with all four waves, in
// the fixed order of the block-summary kernel (so the summary it writes has the
// same bits): its K rows are requested before anything else, since that
// workgroup finishes last.
template <int DT, int D, int G>
__global__ __launch_bounds__(256) void dstep_logits_kernel(DStepArgs a) {
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int DPL = D / 8;
  constexpr int LPR = D / 8, RPP = 256 / LPR;          // refresh: lanes per K row, rows per pass
  constexpr int NV = ES / 2;                           // 16-byte words per lane and K row
  __shared__ float red[RPP][D + 4];
  __shared__ float ered[4][2];
  __shared__ float pooled[D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int row = blockIdx.y, bg = blockIdx.z, b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int jw0 = blockIdx.x * 32 + w * 8;
  const int j = jw0 + (lane >> 3), sub = lane & 7, d0 = sub * DPL;
  const int qpos = a.q_pos0 + row;
  const int nC = a.causal ? min(a.NB, qpos / a.kv_block + 1) : a.NB;
  const bool valid = j < nC;

  // the newest block's first 4 * RPP rows, when this workgroup holds it (uniform over the workgroup)
  const bool ref_wg = a.refresh >= (int)blockIdx.x * 32 && a.refresh < (int)blockIdx.x * 32 + 32 && a.refresh < nC;
  const int rc = tid % LPR, rg = tid / LPR;
  int n_ref = 0;
  const uint8_t* kp = nullptr;
  u32x4 kraw[4][NV];
  if (ref_wg) {
    const int t0 = a.refresh * a.kv_block;
    n_ref = min(a.kv_block, a.L - t0);
    kp = a.k + ((int64_t)b * a.ksb + (int64_t)g * a.ksh + (int64_t)t0 * a.ksl + rc * 8) * ES;
    // rows past the block's end load its last row (zeroed when used): no branch around a load
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = min(u * RPP + rg, n_ref - 1);
#pragma unroll
      for (int c = 0; c < NV; ++c) kraw[u][c] = reinterpret_cast<const u32x4*>(kp + (int64_t)r * a.ksl * ES)[c];
    }
  }

  float qx[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint8_t* qp = a.q + ((int64_t)b * a.qsb + (int64_t)(g * G + h) * a.qsh + (int64_t)row * a.qsl + d0) * ES;
#pragma unroll
    for (int c = 0; c < DPL / 8; ++c) {
      float t[8];
      load8<DT>(qp + c * 8 * ES, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) qx[h][c * 8 + e] = t[e];
    }
  }
  const int64_t mrow = ((int64_t)b * a.Hkv + g) * a.NB;
  float km[DPL];
  if (valid && j != a.refresh) {
    const f32x4* mp = reinterpret_cast<const f32x4*>(a.k_mean + (mrow + j) * D + d0);
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c) {
      const f32x4 t = mp[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) km[4 * c + e] = t[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < DPL; ++e) km[e] = 0.f;
  }
  // the newest block: pooled here from K (Prism sec. 1-2 summary), used and written out
  if (ref_wg) {
    float sum[8], e2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.f;
    auto accumulate = [&](const float (&v)[4][8]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) { sum[e] += v[u][e]; e2 = fmaf(v[u][e], v[u][e], e2); }
    };
    {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = u * RPP + rg < n_ref;
        if constexpr (DT == BSA_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][2 * i] = in ? bf16lo(kraw[u][0][i]) : 0.f;
            v[u][2 * i + 1] = in ? bf16hi(kraw[u][0][i]) : 0.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][i] = in ? __uint_as_float(kraw[u][0][i]) : 0.f;
            v[u][4 + i] = in ? __uint_as_float(kraw[u][NV - 1][i]) : 0.f;
          }
        }
      }
      accumulate(v);
    }
    for (int r0 = 4 * RPP; r0 < n_ref; r0 += 4 * RPP) {                // blocks longer than 4 * RPP rows
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<DT>(kp + (int64_t)min(r0 + u * RPP + rg, n_ref - 1) * a.ksl * ES, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = r0 + u * RPP + rg < n_ref;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = in ? v[u][e] : 0.f;
      }
      accumulate(v);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][rc * 8 + e] = sum[e];
    const int band = band_of_dim(rc * 8, D, a.layout);
    const float ef = wave_sum(band == 0 ? e2 : 0.f), es = wave_sum(band == 0 ? 0.f : e2);
    if (lane == 0) { ered[w][0] = ef; ered[w][1] = es; }
    __syncthreads();
    const float inv = 1.0f / (float)n_ref;
    for (int d = tid; d < D; d += 256) {
      float t = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) t += red[rr][d];
      t *= inv;
      pooled[d] = t;
      if (row == 0) a.k_mean[(mrow + a.refresh) * D + d] = t;
    }
    if (a.k_energy && row == 0 && tid < 2)
      a.k_energy[(mrow + a.refresh) * 2 + tid] = (ered[0][tid] + ered[1][tid] + ered[2][tid] + ered[3][tid]) * inv;
    __syncthreads();
    if (j == a.refresh) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) km[e] = pooled[d0 + e];
    }
  }

  float z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) dot = fmaf(qx[h][e], km[e], dot);
    dot = group_sum<8>(dot);
    z[h] = valid ? dot * a.c2 : -INFINITY;
  }
  const int64_t rowi = ((int64_t)b * a.Hkv + g) * a.Lq + row;
  if (blockIdx.x == 0 && tid == 0) a.arrivals[rowi * 32] = 0u;   // the attention launch counts its slices here
  if (valid) {
    float mine = z[0];
#pragma unroll
    for (int h = 1; h < G; ++h) mine = sub == h ? z[h] : mine;
    if (sub < G) a.Z[(rowi * G + sub) * a.NBp + j] = mine;
  }
  // this wave's softmax partial per head over its 8 blocks
  const int wi = blockIdx.x * 4 + w;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = groups_max<8>(z[h]);
    const float e = m == -INFINITY ? 0.f : fast_exp2(z[h] - m);
    const float l = groups_sum<8>(e);
    if (lane == h) {
      float* st = a.stats + ((rowi * G + h) * a.P + wi) * 2;
      st[0] = m;
      st[1] = l;
    }
  }
}

// -------------------------------------------------------- select + attend ---
template <int DT, int D, int G, int KPL, int NSUB>
__global__ __launch_bounds__(256) void dstep_attend_kernel(DStepArgs a) {
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int KPT = KPL / 4;          // keys per thread: blocks KPT t .. KPT t + KPT - 1
  constexpr int SPL = KPL / 8;          // softmax partials per lane and head (P <= 64 * SPL)
  constexpr int LPT = D / 8;            // lanes per token
  constexpr int TPP = 64 / LPT;         // tokens per wave pass
  constexpr int TPW = kDecTok / 4;      // tokens per wave and sub-chunk
  constexpr int PASSES = TPW / TPP;     // passes per sub-chunk
  constexpr int NP = PASSES * NSUB;     // passes per chunk (NSUB sub-chunks' K/V rows requested at once)
  constexpr int CT = kDecTok * NSUB;    // tokens per chunk
  __shared__ BlockTopkSmem topk_sh;
  __shared__ int32_t lst[64 * KPL];                 // the row's list, ascending
  __shared__ int last_sh;
  __shared__ __attribute__((aligned(16))) uint64_t ml_sh[G * 32];   // the merge's (m, l): [head][slice of the batch]
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_acc[4][G][D];

  const int item = blockIdx.x, row = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int tg = lane / LPT, d0 = (lane % LPT) * 8;
  const int qpos = a.q_pos0 + row;
  const int64_t rowi = ((int64_t)b * a.Hkv + g) * a.Lq + row;
  // candidates, forced blocks and k' of this row (as the selection entry point)
  const int nC = a.causal ? min(a.NB, qpos / a.kv_block + 1) : a.NB;
  const int nf_first = min(a.n_first, nC);
  const int last_lo = max(nf_first, nC - a.n_last);
  const int n_free = last_lo - nf_first;
  int kp = a.topk_num > 0 ? (int)(((int64_t)a.topk_num * nC + a.topk_den - 1) / a.topk_den) : a.topk;
  kp = max(0, min(kp, n_free));

  // ---- loads: queries (for the attention), softmax partials, logits
  float qx[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load8<DT>(a.q + ((int64_t)b * a.qsb + (int64_t)(g * G + h) * a.qsh + (int64_t)row * a.qsl + d0) * ES, qx[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qx[h][e] *= a.c2;
  }
  f32x2 st[G][SPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
      const int pi = lane + 64 * r;
      st[h][r] = pi < a.P ? *reinterpret_cast<const f32x2*>(a.stats + ((rowi * G + h) * a.P + pi) * 2)
                          : f32x2{-INFINITY, 0.f};
    }
  float zv[G][KPT];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < KPT; c += 4) {
      const int j = KPT * tid + c;
      f32x4 z4 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (j < nC) z4 = *reinterpret_cast<const f32x4*>(a.Z + (rowi * G + h) * a.NBp + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) zv[h][c + e] = j + e < nC ? z4[e] : -INFINITY;
    }
  // ---- per-head max and normaliser from the partials (fixed order: the same bits in every wave)
  float Mh[G], invS[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = st[h][0][0];
#pragma unroll
    for (int r = 1; r < SPL; ++r) m = fmaxf(m, st[h][r][0]);
    m = wave_max_dpp(m);
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < SPL; ++r) l += st[h][r][0] == -INFINITY ? 0.f : st[h][r][1] * fast_exp2(st[h][r][0] - m);
    l = wave_sum_dpp(l);
    Mh[h] = m;
    invS[h] = 1.0f / l;
  }
  // ---- group scores as keys (free candidates only; scores >= 0, so float bits order like values)
  uint32_t keys[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int j = KPT * tid + e;
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s = fmaf(fast_exp2(zv[h][e] - Mh[h]), invS[h], s);
    keys[e] = (j >= nf_first && j < last_lo) ? __float_as_uint(s) + 1u : 0u;
  }
  // the list: forced first blocks, the k' best free blocks (ascending), forced newest blocks
  const int np = block_topk<KPT>(keys, kp, n_free, topk_sh, lst + nf_first);
  const int n_list = nf_first + np + (nC - last_lo);
  for (int i = tid; i < nf_first; i += 256) lst[i] = i;
  for (int i = tid; i < nC - last_lo; i += 256) lst[nf_first + np + i] = last_lo + i;
  __syncthreads();
  if (item == 0) {
    for (int i = tid; i < n_list; i += 256) a.idx[rowi * a.cap + i] = lst[i];
    if (tid == 0) a.cnt[rowi] = n_list;
  }

  // ---- attention over this workgroup's slice of the list's tokens
  const int64_t ntok = (int64_t)n_list * a.kv_block;
  const int64_t t_begin = (int64_t)item * a.tok_per_item;
  if (ntok == 0 && item == 0) {                         // nothing selected: O = 0, LSE = -inf
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, d = i - h * D;
      const int64_t oi = (int64_t)b * a.osb + (int64_t)(g * G + h) * a.osh + (int64_t)row * a.osl + d;
      if (a.o_f32) static_cast<float*>(a.o)[oi] = 0.f;
      else static_cast<uint16_t*>(a.o)[oi] = 0;
      if (d == 0) a.lse[((int64_t)b * a.Hkv * G + g * G + h) * a.Lq + row] = -INFINITY;
    }
  }
  if (t_begin >= ntok) return;                          // no slice of the list for this workgroup
  const int64_t t_end = min(ntok, t_begin + a.tok_per_item);
  if constexpr (NSUB > 1 && DT == BSA_BF16 && D == 128) {
    // lengthened slices (many lists in one launch): scores on the matrix cores, as the attention
    // entry point's form for such launches (dec_wide_chunk), the list from LDS.  (On 32-token
    // slices the vector form below is faster here: measured 16.9 against 17.5 us per 64K step.)
    constexpr int GP = G < 4 ? 4 : G;
    __shared__ __attribute__((aligned(16))) float p_sh[4][32][GP];
    __shared__ float al_sh[4][G];
    const int col = lane & 15, kq = lane >> 4;
    const int hq = g * G + min(col, G - 1);           // columns past G load a valid row, then zeroed
    bf16x8 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 qw = *reinterpret_cast<const u32x4*>(
          a.q + ((int64_t)b * a.qsb + (int64_t)hq * a.qsh + (int64_t)row * a.qsl + 32 * ks + 8 * kq) * 2);
      qb[ks] = __builtin_bit_cast(bf16x8, col < G ? qw : u32x4{0u, 0u, 0u, 0u});
    }
    float m_run = -INFINITY, l_run = 0.f, acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    const uint8_t* kbw = a.k + ((int64_t)b * a.ksb + (int64_t)g * a.ksh) * 2;
    const uint8_t* vbw = a.v + ((int64_t)b * a.vsb + (int64_t)g * a.vsh) * 2;
    for (int64_t c0 = t_begin; c0 < t_end; c0 += CT) {
      const int64_t tw = c0 + 32 * w;                 // the wave's first token
      // the lane's K rows (key col of each 16-key half) and V rows (tokens 4 rd + kq); list tokens < 2^31
      int pos[10];
      bool ok[10];
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        const int64_t t = j < 2 ? tw + 16 * j + col : tw + 4 * (j - 2) + kq;
        const bool in = t < t_end;
        const int e = in ? (int)((uint32_t)t / (uint32_t)a.kv_block) : 0;
        const int blk = in ? lst[e] : -1;
        const int64_t key = (int64_t)blk * a.kv_block + (t - (int64_t)e * a.kv_block);
        ok[j] = in && blk >= 0 && key < a.L && (!a.causal || key <= qpos);
        pos[j] = ok[j] ? (int)key : 0;
      }
      bf16x8 kf[2][4];
      u32x4 vr[8];
      bool kok[2], vok[8];
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        kok[kg] = ok[kg];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kf[kg][ks] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kbw + ((int64_t)pos[kg] * a.ksl + 32 * ks + 8 * kq) * 2));
      }
#pragma unroll
      for (int rd = 0; rd < 8; ++rd) {
        vok[rd] = ok[2 + rd];
        vr[rd] = *reinterpret_cast<const u32x4*>(vbw + ((int64_t)pos[2 + rd] * a.vsl + 8 * col) * 2);
      }
      dec_wide_chunk<G>(qb, kf, vr, kok, vok, a.c2, m_run, l_run, acc, p_sh[w], al_sh[w]);
    }
    // the four token sets summed; row 0 of the wave holds dims 8 col .. 8 col + 7
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = groups_sum<16>(acc[h][e]);
    if (kq == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[w][h][8 * col + e] = acc[h][e];
      if (col < G) { sm_m[w][col] = m_run; sm_l[w][col] = l_run; }
    }
  } else {
    float wm[G], wl[G], wacc[G][8];
  #pragma unroll
    for (int h = 0; h < G; ++h) {
      wm[h] = -INFINITY;
      wl[h] = 0.f;
  #pragma unroll
      for (int e = 0; e < 8; ++e) wacc[h][e] = 0.f;
    }
    const uint8_t* kb = a.k + ((int64_t)b * a.ksb + (int64_t)g * a.ksh + d0) * ES;
    const uint8_t* vb = a.v + ((int64_t)b * a.vsb + (int64_t)g * a.vsh + d0) * ES;
    for (int64_t c0 = t_begin; c0 < t_end; c0 += CT) {
      int pos[NP];
      bool ok[NP];
  #pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int64_t t = c0 + (p / PASSES) * kDecTok + w * TPW + (p % PASSES) * TPP + tg;
        const bool in = t < t_end;
        const int e = in ? (int)((uint32_t)t / (uint32_t)a.kv_block) : 0;   // list tokens < 2^31
        const int blk = in ? lst[e] : -1;
        const int64_t key = (int64_t)blk * a.kv_block + (t - (int64_t)e * a.kv_block);
        ok[p] = in && blk >= 0 && key < a.L && (!a.causal || key <= qpos);
        pos[p] = ok[p] ? (int)key : 0;
      }
      // every pass loads (row 0 stands in for a masked token, zeroed when widened): a load under a
      // branch would make the compiler wait for one pass's rows before requesting the next
      Raw8<DT> kr[NP], vr[NP];
  #pragma unroll
      for (int p = 0; p < NP; ++p) {
        kr[p] = load_raw8<DT>(kb + (int64_t)pos[p] * a.ksl * ES);
        vr[p] = load_raw8<DT>(vb + (int64_t)pos[p] * a.vsl * ES);
      }
  #pragma unroll
      for (int sc = 0; sc < NSUB; ++sc) {
        // a sub-chunk past the slice's end has no visible token and leaves the state as it is
        Raw8<DT> ks[PASSES], vs[PASSES];
        bool oks[PASSES];
  #pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          ks[p] = kr[sc * PASSES + p];
          vs[p] = vr[sc * PASSES + p];
          oks[p] = ok[sc * PASSES + p];
        }
        dec_sub_chunk<DT, D, G, PASSES>(qx, ks, vs, oks, wm, wl, wacc);
      }
    }
  #pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane < LPT) {
  #pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[w][h][d0 + e] = wacc[h][e];
      }
      if (lane == 0) { sm_m[w][h] = wm[h]; sm_l[w][h] = wl[h]; }
    }
  }
  __syncthreads();
  // merge the 4 waves into this workgroup's partial, stored at device scope (no cache holds it back)
  const int64_t pbase = (rowi * a.items + item) * G;
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, d = i - h * D;
    float M = sm_m[0][h];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][h]);
    float o = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        if (sm_m[ww][h] == -INFINITY) continue;
        const float wgt = fast_exp2(sm_m[ww][h] - M);
        o = fmaf(sm_acc[ww][h][d], wgt, o);
        lsum = fmaf(sm_l[ww][h], wgt, lsum);
      }
    }
    st_dev(a.part_o + (pbase + h) * D + d, o);
    if (d == 0) st_dev2(a.part_ml + (pbase + h) * 2, M, lsum);
  }
  const int n_valid = (int)((ntok + a.tok_per_item - 1) / a.tok_per_item);
  if (!arrive_last(a.arrivals + rowi * 32, n_valid, last_sh)) return;
  // the last slice to finish merges all slices in order
  merge_published<G, D>(a.part_o + rowi * a.items * G * D, a.part_ml + rowi * a.items * G * 2, n_valid, ml_sh,
                        a.o, a.o_f32, (int64_t)b * a.osb + (int64_t)(g * G) * a.osh + (int64_t)row * a.osl, a.osh,
                        a.lse + ((int64_t)b * a.Hkv * G + g * G) * a.Lq + row, a.Lq);
}

// ------------------------------------------------------------------- host ---
bool plan_decode_step(const bsa_tensor& q, const bsa_tensor& k, const bsa_select_params& p, DStepPlan& pl) {
  pl.B = q.B;
  pl.Hq = q.H;
  pl.Hkv = k.H;
  pl.G = q.H / k.H;
  pl.D = q.D;
  pl.Lq = q.L;
  pl.L = k.L;
  pl.NB = (int)ceil_div(k.L, p.kv_block);
  pl.NBp = (pl.NB + 3) & ~3;
  pl.KPL = pl.NB <= 1024 ? 16 : 64;
  pl.P = 4 * (int)ceil_div(pl.NB, 32);
  const int64_t toks = (int64_t)p.cap * p.kv_block;
  pl.tok_per_item = (int)dec_slice_tokens(toks, (int64_t)pl.B * pl.Hkv * pl.Lq);
  pl.items = (int)ceil_div(toks, pl.tok_per_item);
  const size_t rows = (size_t)pl.B * pl.Hkv * pl.Lq;
  pl.z_bytes = align256(rows * pl.G * pl.NBp * 4);
  pl.stats_bytes = align256(rows * pl.G * pl.P * 2 * 4);
  pl.part_o_bytes = align256(rows * pl.items * pl.G * pl.D * 4);
  pl.part_ml_bytes = align256(rows * pl.items * pl.G * 2 * 4);
  pl.arrival_bytes = align256(rows * 32 * 4);
  return true;
}

void launch_decode_step(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, float* k_mean,
                        float* k_energy, int refresh, const bsa_select_params& p, const DStepPlan& pl, int32_t* idx,
                        int32_t* cnt, const bsa_tensor& o, float* lse, void* ws, hipStream_t s) {
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  DStepArgs a;
  a.q = static_cast<const uint8_t*>(q.data);
  a.k = static_cast<const uint8_t*>(k.data);
  a.v = static_cast<const uint8_t*>(v.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
  a.k_mean = k_mean; a.k_energy = k_energy; a.refresh = refresh;
  a.B = pl.B; a.Hkv = pl.Hkv; a.Lq = pl.Lq; a.L = pl.L; a.NB = pl.NB; a.NBp = pl.NBp;
  a.kv_block = p.kv_block; a.q_pos0 = p.q_pos0; a.causal = p.causal; a.layout = p.layout;
  a.topk = p.topk; a.topk_num = p.topk_num; a.topk_den = p.topk_den; a.n_first = p.n_first; a.n_last = p.n_last;
  a.cap = p.cap;
  a.c2 = p.scale * kLog2e;
  a.Z = reinterpret_cast<float*>(w8);
  a.stats = reinterpret_cast<float*>(w8 + pl.z_bytes);
  a.P = pl.P;
  a.idx = idx; a.cnt = cnt;
  a.part_o = reinterpret_cast<float*>(w8 + pl.z_bytes + pl.stats_bytes);
  a.part_ml = reinterpret_cast<float*>(w8 + pl.z_bytes + pl.stats_bytes + pl.part_o_bytes);
  a.arrivals = reinterpret_cast<uint32_t*>(w8 + pl.z_bytes + pl.stats_bytes + pl.part_o_bytes + pl.part_ml_bytes);
  a.items = pl.items; a.tok_per_item = pl.tok_per_item;
  a.o = o.data; a.o_f32 = o.dtype == BSA_F32; a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
  a.lse = lse;

  const dim3 g1((unsigned)ceil_div(pl.NB, 32), (unsigned)pl.Lq, (unsigned)(pl.B * pl.Hkv));
  const dim3 g2((unsigned)pl.items, (unsigned)pl.Lq, (unsigned)(pl.B * pl.Hkv));
  const bool wide = pl.tok_per_item % (kDecTok * kDecWideSub) == 0;
#define BSA_DS_ATT(DT, DD, GG, KK)                                                                                  \
  do {                                                                                                             \
    if (wide) hipLaunchKernelGGL((dstep_attend_kernel<DT, DD, GG, KK, kDecWideSub>), g2, dim3(256), 0, s, a);    \
    else hipLaunchKernelGGL((dstep_attend_kernel<DT, DD, GG, KK, 1>), g2, dim3(256), 0, s, a);                   \
  } while (0)
#define BSA_DS(DT, DD, GG)                                                                                  \
  do {                                                                                                     \
    hipLaunchKernelGGL((dstep_logits_kernel<DT, DD, GG>), g1, dim3(256), 0, s, a);                          \
    if (pl.KPL == 16) BSA_DS_ATT(DT, DD, GG, 16);                                                           \
    else BSA_DS_ATT(DT, DD, GG, 64);                                                                        \
  } while (0)
#define BSA_DS_G(DT, DD)                       \
  do {                                         \
    switch (pl.G) {                            \
      case 1: BSA_DS(DT, DD, 1); break;        \
      case 2: BSA_DS(DT, DD, 2); break;        \
      case 4: BSA_DS(DT, DD, 4); break;        \
      default: BSA_DS(DT, DD, 8); break;       \
    }                                          \
  } while (0)
  if (q.dtype == BSA_BF16) {
    if (pl.D == 128) BSA_DS_G(BSA_BF16, 128); else BSA_DS_G(BSA_BF16, 64);
  } else {
    if (pl.D == 128) BSA_DS_G(BSA_F32, 128); else BSA_DS_G(BSA_F32, 64);
  }
#undef BSA_DS_G
#undef BSA_DS
#undef BSA_DS_ATT

}

}  // namespace bsa
