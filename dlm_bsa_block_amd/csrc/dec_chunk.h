// One decode sub-chunk of kDecTok list tokens: the arithmetic shared by the
// decode attention kernel and the decode step's attention, so that both give
// the same bits for the same list.
//
// Layout of the work (D = 128: 16 lanes per token, 4 tokens per wave pass; a
// wave takes kDecTok / 4 tokens of a sub-chunk in PASSES passes): each lane
// holds 8 consecutive dims of its token's K and V row.  K and V are loaded as
// raw storage words and widened only where a sub-chunk is computed, so a
// workgroup can request several sub-chunks' rows at once (one memory round
// trip for all of them) without holding them as floats.
#pragma once
#include "common.h"
#include "split.h"

namespace bsa {

template <int DT>
struct Raw8;
template <>
struct Raw8<BSA_BF16> {
  u32x4 w;
};
template <>
struct Raw8<BSA_F32> {
  f32x4 a, b;
};

// 8 consecutive elements, 16-byte aligned, as stored
template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw8(const void* p) {
  Raw8<DT> r;
  if constexpr (DT == BSA_BF16) {
    r.w = *reinterpret_cast<const u32x4*>(p);
  } else {
    r.a = reinterpret_cast<const f32x4*>(p)[0];
    r.b = reinterpret_cast<const f32x4*>(p)[1];
  }
  return r;
}

// widen to floats; a token that is not visible gets zeros
template <int DT>
__device__ __forceinline__ void widen8(const Raw8<DT>& r, bool ok, float (&o)[8]) {
  if constexpr (DT == BSA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = ok ? bf16lo(r.w[i]) : 0.f;
      o[2 * i + 1] = ok ? bf16hi(r.w[i]) : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = ok ? r.a[i] : 0.f;
      o[4 + i] = ok ? r.b[i] : 0.f;
    }
  }
}

// Online-softmax update of one wave's running state (wm, wl, wacc per head,
// log2 units) with the PASSES passes of one sub-chunk: per head, the scores of
// the wave's tokens (q pre-scaled by scale * log2 e), their maximum over the
// wave, p = 2^(s - m_new), and the p-weighted sums of l and V, all reduced over
// the wave's tokens in a fixed order.
template <int DT, int D, int G, int PASSES>
__device__ __forceinline__ void dec_sub_chunk(const float (&qx)[G][8], const Raw8<DT> (&kr)[PASSES],
                                              const Raw8<DT> (&vr)[PASSES], const bool (&ok)[PASSES],
                                              float (&wm)[G], float (&wl)[G], float (&wacc)[G][8]) {
  constexpr int LPT = D / 8;            // lanes per token
  float kx[PASSES][8], vx[PASSES][8];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    widen8<DT>(kr[p], ok[p], kx[p]);
    widen8<DT>(vr[p], ok[p], vx[p]);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qx[h][e], kx[p][e], dot);
      dot = group_sum<LPT>(dot);
      s[p] = ok[p] ? dot : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int p = 1; p < PASSES; ++p) mx = fmaxf(mx, s[p]);
    mx = groups_max<LPT>(mx);
    const float m_new = fmaxf(wm[h], mx);
    if (m_new == -INFINITY) continue;                  // nothing visible yet (wave-uniform)
    const float alpha = fast_exp2(wm[h] - m_new);
    float l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float pr = ok[p] ? fast_exp2(s[p] - m_new) : 0.f;
      l += pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pr, vx[p][e], acc[e]);
    }
    l = groups_sum<LPT>(l);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = groups_sum<LPT>(acc[e]);
    wm[h] = m_new;
    wl[h] = fmaf(wl[h], alpha, l);
#pragma unroll
    for (int e = 0; e < 8; ++e) wacc[h][e] = fmaf(wacc[h][e], alpha, acc[e]);
  }
}

// One chunk of 32 keys per wave on the matrix cores (bf16, D = 128): the keys'
// scores S^T = K Q^T (16 keys x 16 query columns per v_mfma_f32_16x16x32_bf16;
// the A operand's lane l holds key l & 15, dims 32 ks + 8 (l >> 4) + 0..7), the
// online-softmax update of the head's running (m, l) held by the lanes of
// column h, and acc[h][e] += p v over the lane's 8 tokens 4 rd + (l >> 4) at
// dims 8 (l & 15) + e.  qb: the Q^T operand (columns past G zero); kok: the
// validity of key l & 15 in each 16-key half; vok: of the lane's V tokens.
// p_w (32 x GP floats) and al_w (G floats) are the wave's LDS exchange area.
template <int G, int GP = (G < 4 ? 4 : G)>
__device__ __forceinline__ void dec_wide_chunk(const bf16x8 (&qb)[4], const bf16x8 (&kf)[2][4], const u32x4 (&vr)[8],
                                               const bool (&kok)[2], const bool (&vok)[8], float c2, float& m_run,
                                               float& l_run, float (&acc)[G][8], float (*p_w)[GP], float* al_w) {
  const int lane = threadIdx.x & 63, col = lane & 15, kq = lane >> 4;
  // scores: lane holds keys 16 kg + 4 kq + r of head col; key validity from the A-row lanes' ballot
  float sv[2][4];
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const uint32_t okm = (uint32_t)__builtin_amdgcn_ballot_w64(kok[kg]) & 0xFFFFu;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kg][ks], qb[ks], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[kg][r] = (okm >> (4 * kq + r)) & 1u ? c[r] * c2 : -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                   fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
  mt = groups_max<16>(mt);                            // over the four key quads: the head's max
  const float m_new = fmaxf(m_run, mt);
  const float msub = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2(m_run - msub);        // 0 while nothing was visible
  float lt = 0.f;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[kg][r] = fast_exp2(sv[kg][r] - msub);        // p; 0 for a masked key
      lt += sv[kg][r];
    }
  lt = groups_sum<16>(lt);
  l_run = fmaf(l_run, alpha, lt);
  m_run = m_new;
  if (col < G) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int r = 0; r < 4; ++r) p_w[16 * kg + 4 * kq + r][col] = sv[kg][r];
    if (kq == 0) al_w[col] = alpha;
  }
  wave_sync_lds();
  // P V: rescale, then the lane's 8 tokens (4 rd + kq) in order
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float al = al_w[h];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] *= al;
  }
#pragma unroll
  for (int rd = 0; rd < 8; ++rd) {
    float pj[GP];
#pragma unroll
    for (int h4 = 0; h4 < GP; h4 += 4) {
      const f32x4 t4 = *reinterpret_cast<const f32x4*>(&p_w[4 * rd + kq][h4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) pj[h4 + e] = t4[e];
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = vok[rd] ? bf16lo(vr[rd][i]) : 0.f;
      v[2 * i + 1] = vok[rd] ? bf16hi(vr[rd][i]) : 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pj[h], v[e], acc[h][e]);
  }
  wave_sync_lds();                                    // p_w is rewritten by the next chunk
}

}  // namespace bsa
