// Top-k' selection of block scores inside one wavefront, with no LDS atomics,
// no workgroup barriers and few scalar round trips (a dependent chain of
// vector compare -> scalar count -> vector compare costs tens of cycles a
// step here, so the work is shaped as independent vector operations).
//
// Keys are uint32 with a larger key a better block (the bits of a
// non-negative fp32 score plus one); 0 marks a block that is not a free
// candidate.  Lane l holds the keys of blocks j = KPL l + e, e < KPL, so lane
// order is block order.  The k' best keys are taken, ties at the k'-th key
// going to the lower block index.
//
// The k'-th largest key T is found in two steps when k' <= 64.  The lanes'
// maxima are sorted across the wave (a bitonic network of lane exchanges);
// the k'-th of them, T0, has at least k' keys at or above it (the k' lanes
// whose maximum reaches it), so T >= T0 and every key >= T is among the n0
// keys >= T0.  When n0 <= 64 those keys are gathered one per lane and each
// lane counts the gathered keys that outrank its own: the key of rank k' - 1
// is T.  Otherwise (or when k' > 64) T is found bit by bit from the top.
// A last pass flags the keys above T and, of the keys equal to T, the first
// k' - #{keys > T} in block order.
#pragma once
#include "common.h"

namespace bsa {

// Value of lane l ^ J (J a power of two below 64).
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  if constexpr (J == 1) return dpp_u32<0xB1>(0u, v);                 // quad_perm [1,0,3,2]
  else if constexpr (J == 2) return dpp_u32<0x4E>(0u, v);            // quad_perm [2,3,0,1]
  else if constexpr (J == 4) {
    const uint32_t up = dpp_u32<0x12C>(0u, v), dn = dpp_u32<0x124>(0u, v);   // row_ror 12 / 4: lane +4 / -4
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) return dpp_u32<0x128>(0u, v);         // row_ror 8
  else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v) {
  const uint32_t o = lane_xor_u32<J>(v);
  const int lane = threadIdx.x & 63;
  const bool desc = (lane & K) == 0, lower = (lane & J) == 0;
  return (lower == desc) ? max(v, o) : min(v, o);
}

// The 64 lanes' values sorted in descending order (lane 0 the largest).
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v) {
  v = bitonic_step<2, 1>(v);
  v = bitonic_step<4, 2>(v);  v = bitonic_step<4, 1>(v);
  v = bitonic_step<8, 4>(v);  v = bitonic_step<8, 2>(v);  v = bitonic_step<8, 1>(v);
  v = bitonic_step<16, 8>(v); v = bitonic_step<16, 4>(v); v = bitonic_step<16, 2>(v); v = bitonic_step<16, 1>(v);
  v = bitonic_step<32, 16>(v); v = bitonic_step<32, 8>(v); v = bitonic_step<32, 4>(v);
  v = bitonic_step<32, 2>(v);  v = bitonic_step<32, 1>(v);
  v = bitonic_step<64, 32>(v); v = bitonic_step<64, 16>(v); v = bitonic_step<64, 8>(v);
  v = bitonic_step<64, 4>(v);  v = bitonic_step<64, 2>(v);  v = bitonic_step<64, 1>(v);
  return v;
}

__device__ __forceinline__ uint32_t lane_read(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// The kp-th largest of all keys (with repeats), bit by bit from the top.
template <int KPL>
__device__ __forceinline__ uint32_t wave_kth_largest_n(const uint32_t (&k)[KPL], int kp) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int n = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) n += (int)__popcll(__ballot(k[i] >= c));
    if (n >= kp) t = c;
  }
  return t;
}

// Flags of one selection row's picks: bit e of the result is set when block
// KPL * lane + e is among the kp best free candidates (kp, n_free
// wave-uniform; n_free = number of nonzero keys).  cand: 64 words of LDS owned
// by this wavefront.  Every lane of the wave must call it.
template <int KPL>
__device__ uint64_t wave_topk(const uint32_t (&k)[KPL], int kp, int n_free, uint32_t* cand) {
  static_assert(KPL >= 1 && KPL <= 64, "keys per lane");
  const int lane = threadIdx.x & 63;
  uint64_t sel = 0;
  if (kp <= 0) return 0;
  if (kp >= n_free) {
#pragma unroll
    for (int e = 0; e < KPL; ++e)
      if (k[e] != 0u) sel |= 1ull << e;
    return sel;
  }
  uint32_t T = 0;
  bool found = false;
  if (kp <= 64) {
    uint32_t mx = k[0];
#pragma unroll
    for (int e = 1; e < KPL; ++e) mx = max(mx, k[e]);
    const uint32_t t0 = max(1u, lane_read(wave_sort_desc(mx), kp - 1));
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) c += k[e] >= t0 ? 1u : 0u;
    const uint32_t incl = wave_incl_scan_dpp(c);
    const int n0 = (int)lane_read(incl, 63);
    if (n0 <= 64) {
      int pos = (int)(incl - c);
      cand[lane] = 0u;                       // slots past n0 stay 0: below every gathered key
      wave_sync_lds();
#pragma unroll
      for (int e = 0; e < KPL; ++e)
        if (k[e] >= t0) cand[pos++] = k[e];
      wave_sync_lds();
      const uint32_t mine = cand[lane];
      // rank = keys that outrank this one: larger, or equal and earlier in block order (a zero
      // slot outranks no gathered key).  The slots are read 32 at a time, all requested before
      // the first compare.
      int rank = 0;
      for (int m0 = 0; m0 < n0; m0 += 32) {
        u32x4 q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = *reinterpret_cast<const u32x4*>(cand + m0 + 4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int m = m0 + 4 * i + t;
            rank += (q[i][t] > mine) ? 1 : 0;
            rank += (q[i][t] == mine && m < lane) ? 1 : 0;
          }
      }
      const uint64_t at = __ballot(lane < n0 && rank == kp - 1);
      T = lane_read(mine, __ffsll((unsigned long long)at) - 1);
      found = true;
      wave_sync_lds();                       // cand may be rewritten by the caller's next row
    }
  }
  if (!found) T = wave_kth_largest_n<KPL>(k, kp);
  // keys above T are all taken; of the keys equal to T the first (in block order) kp - #{> T}
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    gt += k[e] > T ? 1u : 0u;
    eq += k[e] == T ? 1u : 0u;
  }
  const int need = kp - (int)lane_read(wave_incl_scan_dpp(gt), 63);
  int r = (int)(wave_incl_scan_dpp(eq) - eq);       // equal keys in earlier lanes
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    if (k[e] > T) sel |= 1ull << e;
    else if (k[e] == T) {
      if (r < need) sel |= 1ull << e;
      ++r;
    }
  }
  return sel;
}

// Ascending list of the flagged blocks (bit e on lane l = block KPL l + e),
// written to out[0 .. n) and padded with -1 up to pad_to; returns n
// (wave-uniform).  One wavefront.
template <int KPL>
__device__ __forceinline__ int wave_flags_to_list(uint64_t flags, int32_t* out, int pad_to) {
  const int lane = threadIdx.x & 63;
  const uint32_t c = (uint32_t)__popcll(flags);
  const uint32_t incl = wave_incl_scan_dpp(c);
  int pos = (int)(incl - c);
  uint64_t f = flags;
  while (f) {
    const int e = __ffsll((unsigned long long)f) - 1;
    f &= f - 1;
    out[pos++] = KPL * lane + e;
  }
  const int n = (int)lane_read(incl, 63);
  for (int p = n + lane; p < pad_to; p += 64) out[p] = -1;
  return n;
}

// The flags as a bitmap of 32-bit words (word w covers blocks 32 w .. 32 w + 31),
// words [0, nwords) written; one wavefront.
template <int KPL>
__device__ __forceinline__ void wave_flags_to_bits(uint64_t flags, uint32_t* out, int nwords) {
  const int lane = threadIdx.x & 63;
  if constexpr (KPL >= 32) {
#pragma unroll
    for (int h = 0; h < KPL / 32; ++h) {
      const int wd = lane * (KPL / 32) + h;
      if (wd < nwords) out[wd] = (uint32_t)(flags >> (32 * h));
    }
  } else {
    // 32 / KPL lanes per word: OR their shifted masks together across the lanes of the word
    constexpr int LPW = 32 / KPL;
    uint32_t v = (uint32_t)flags << (KPL * (lane % LPW));
    if constexpr (LPW >= 2) v |= lane_xor_u32<1>(v);
    if constexpr (LPW >= 4) v |= lane_xor_u32<2>(v);
    if constexpr (LPW >= 8) v |= lane_xor_u32<4>(v);
    if constexpr (LPW >= 16) v |= lane_xor_u32<8>(v);
    if constexpr (LPW >= 32) v |= lane_xor_u32<16>(v);
    const int wd = lane / LPW;
    if (lane % LPW == 0 && wd < nwords) out[wd] = v;
  }
}

}  // namespace bsa

namespace bsa {

// ---------------------------------------------------------------------------
// The same selection over a workgroup of 256 threads, thread t holding the
// keys of blocks KPT t + e (e < KPT): each wave sorts its lanes' maxima and
// offers the k'-th of them; the largest offer T0 bounds T from below.  The
// keys >= T0 (with their block index, so that ties order by block) are
// gathered in LDS and each one counts the gathered keys that outrank it; the
// one of rank k' - 1 is T.  Block-order prefix counts of the keys above and
// equal to T then place every pick directly at its position in the ascending
// list.  Four barriers; no thread does more than KPT + the gathered count
// compares.  The gathering appends with one LDS atomicAdd per wave; the order
// in which the waves append does not matter, since the ranks come from the
// unique (key, index) pairs.
struct __attribute__((aligned(16))) BlockTopkSmem {
  uint64_t cand[256];                 // first: read 16 bytes at a time
  uint32_t offer[4];
  uint32_t gt[4], eq[4];
  uint32_t n_cand;
  uint32_t T;
};

// Writes the picks (ascending block index) to out[0 .. n) and returns n =
// min(kp, n_free) (uniform).  kp and n_free (the number of nonzero keys) are
// uniform over the workgroup; every thread must call it; the caller
// synchronises before reading out.
template <int KPT>
__device__ int block_topk(const uint32_t (&k)[KPT], int kp, int n_free, BlockTopkSmem& sm, int32_t* out) {
  // one workgroup of 256 threads: thread t holds the keys of blocks KPT t .. KPT t + KPT - 1
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (kp <= 0 || n_free <= 0) return 0;
  uint32_t T = 0;                                      // with T = 0 every free key is "above"
  if (kp < n_free) {
    if (t == 0) sm.n_cand = 0u;
    sm.cand[t] = 0u;                                   // below every gathered key: the rank loop reads past n0
    uint32_t t0 = 1u;
    if (kp <= 64) {
      uint32_t mx = k[0];
#pragma unroll
      for (int e = 1; e < KPT; ++e) mx = max(mx, k[e]);
      // read in converged code: a lane read inside a branch may see a lane the branch left inactive
      const uint32_t offer = lane_read(wave_sort_desc(mx), kp - 1);
      if (lane == 0) sm.offer[w] = offer;
    }
    __syncthreads();
    if (kp <= 64) t0 = max(1u, max(max(sm.offer[0], sm.offer[1]), max(sm.offer[2], sm.offer[3])));
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) c += k[e] >= t0 ? 1u : 0u;
    const uint32_t incl = wave_incl_scan_dpp(c);
    uint32_t base = 0;
    if (lane == 63) base = atomicAdd(&sm.n_cand, incl);
    base = lane_read(base, 63) + incl - c;
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      if (k[e] >= t0) {
        if (base < 256u) sm.cand[base] = ((uint64_t)k[e] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(KPT * t + e));
        ++base;
      }
    __syncthreads();
    const int n0 = (int)sm.n_cand;
    if (n0 <= 256) {
      // composite keys are unique: rank = gathered keys that outrank this one
      if (t < n0) {
        const uint64_t mine = sm.cand[t];
        int rank = 0;
        // eight keys per round, four 16-byte reads in flight; slots past n0 hold 0
        for (int m0 = 0; m0 < n0; m0 += 8) {
          u32x4 q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) q[r] = *reinterpret_cast<const u32x4*>(&sm.cand[m0 + 2 * r]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint64_t a = (uint64_t)q[r][0] | ((uint64_t)q[r][1] << 32);
            const uint64_t b = (uint64_t)q[r][2] | ((uint64_t)q[r][3] << 32);
            rank += (a > mine ? 1 : 0) + (b > mine ? 1 : 0);
          }
        }
        if (rank == kp - 1) sm.T = (uint32_t)(mine >> 32);
      }
      __syncthreads();
      T = sm.T;
    } else {
      // many keys near the k'-th (ties, flat scores): T bit by bit from the top, counted over the workgroup
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cnd = T | (1u << bit);
        uint32_t cc = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) cc += k[e] >= cnd ? 1u : 0u;
        cc = lane_read(wave_incl_scan_dpp(cc), 63);
        if (lane == 0) sm.gt[w] = cc;
        __syncthreads();
        const uint32_t tot = sm.gt[0] + sm.gt[1] + sm.gt[2] + sm.gt[3];
        __syncthreads();
        if ((int)tot >= kp) T = cnd;
      }
    }
  }
  // block-order prefix counts of the keys above and equal to T
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    gt += k[e] > T ? 1u : 0u;
    eq += (T != 0u && k[e] == T) ? 1u : 0u;
  }
  const uint32_t gi = wave_incl_scan_dpp(gt), ei = wave_incl_scan_dpp(eq);
  if (lane == 63) { sm.gt[w] = gi; sm.eq[w] = ei; }
  __syncthreads();
  uint32_t gtb = gi - gt, eqb = ei - eq, gtot = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    gtot += sm.gt[ww];
    if (ww < w) { gtb += sm.gt[ww]; eqb += sm.eq[ww]; }
  }
  const uint32_t need = kp > (int)gtot ? (uint32_t)kp - gtot : 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int j = KPT * t + e;
    if (k[e] > T) {
      out[gtb + min(eqb, need)] = j;
      ++gtb;
    } else if (T != 0u && k[e] == T) {
      if (eqb < need) out[gtb + eqb] = j;
      ++eqb;
    }
  }
  return kp < n_free ? kp : n_free;
}

}  // namespace bsa
