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

}  // namespace bsa
