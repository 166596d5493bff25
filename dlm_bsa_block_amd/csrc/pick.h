// Arguments and per-row plan of the block pick (top-k' of the group scores
// plus the forced blocks, NSA page's selection setting; scores from the
// pooled-key logits, Prism page sec. 1), shared by the selection kernels and
// the denoising step, which picks inside its attention launch.
#pragma once
#include "common.h"
#include "internal.h"
#include "wave_select.h"

namespace bsa {

struct PickArgs {
  const float* Z;
  int NB, NBp, Rtot, G, Hkv, nbands, NQB;
  int q_block, kv_block, q_pos0, Lq, causal, pooled;
  int multi_row;           // raw rows with more than one row per query block: rows publish bitmaps
  int topk, topk_num, topk_den, n_first, n_last, cap;
  const uint8_t* row_mask;
  int32_t* idx;
  int32_t* cnt;
  int32_t* row_picks;
  uint32_t* row_bits;      // [B][Hkv][Rtot][128] row bitmaps (blocks with several rows)
};

constexpr int kPickMaxWords = 128;     // NB <= 4096
constexpr int kPickThreads = 256;
constexpr int kPickRegs = 32;          // logits held per thread at once
constexpr int kPickChanBatch = 16;     // (head, band) channels reduced together, at most

struct RowPlan {
  int qb, rows, nC, nf_first, last_lo, kp, n_free;
};

__device__ __forceinline__ RowPlan row_plan(const PickArgs& a, int row) {
  RowPlan r;
  r.qb = a.pooled ? row : row / a.q_block;
  r.rows = a.pooled ? 1 : min(a.q_block, a.Lq - r.qb * a.q_block);
  int jmax = a.NB - 1;
  if (a.causal) {
    const int last_row = min((r.qb + 1) * a.q_block, a.Lq) - 1;
    jmax = min(a.NB - 1, (a.q_pos0 + last_row) / a.kv_block);
  }
  r.nC = jmax + 1;
  r.nf_first = min(a.n_first, r.nC);
  r.last_lo = max(r.nf_first, r.nC - a.n_last);       // forced: j < nf_first or j >= last_lo
  const int n_forced = r.nf_first + (r.nC - r.last_lo);
  int kp = a.topk_num > 0 ? (int)(((int64_t)a.topk_num * r.nC + a.topk_den - 1) / a.topk_den) : a.topk;
  r.kp = max(0, min(kp, r.nC - n_forced));
  r.n_free = r.nC - n_forced;
  return r;
}


// The pick arguments of a selection (Z, the row bitmaps and the list outputs in the selection
// workspace layout of plan_select).
PickArgs make_pick_args(const bsa_select_params& p, const SelectPlan& pl, void* ws, const uint8_t* row_mask,
                        int32_t* idx, int32_t* cnt, int32_t* row_picks);

// The denoising step's split gather (one query block of R rows): each workgroup picks the active
// rows' blocks from the logits in pk.Z, takes the union (written to idx / cnt by workgroup 0) and
// attends to its slice of it, writing split partials to ws (the attention workspace layout).
void launch_denoise_gather(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const bsa_attn_params& p,
                           const AttnPlan& pl, const PickArgs& pk, const uint8_t* row_mask, int32_t* idx,
                           int32_t* cnt, void* ws, hipStream_t s);

// The picks of one selection row by a single wavefront, with the arithmetic of
// the 256-thread pick of the selection entry point: lane l stands for the
// threads 64 v + l (v < 4) of that workgroup, which own the candidates
// j = 64 v + l + 256 u.  Each per-thread sum is formed in the same order, the
// four of a lane are added in order of v and the lane sums go through the same
// DPP network (block_sum_lanes_n there; the maxima, exact in any order, take
// one reduction), so every score, and hence every pick, has the same bits.  keys: 256 U words of LDS and cand: 64 words, both owned by this
// wavefront.  Returns the flags of blocks KPL lane + e (KPL = 4 U), forced
// blocks included.
template <int U>
__device__ uint64_t wave_pick_row(const PickArgs& a, int b, int g, int row, uint32_t* keys, uint32_t* cand) {
  constexpr int KPL = 4 * U;
  constexpr int CW = (8 / U) > 0 ? 8 / U : 1;       // channels loaded together (32 values a lane)
  const int lane = threadIdx.x & 63;
  const RowPlan rp = row_plan(a, row);
  const int nC = rp.nC, NBp = a.NBp, nchan = a.G * a.nbands;
  const float* zrow = a.Z + (((int64_t)b * a.Hkv + g) * a.Rtot + row) * (int64_t)nchan * NBp;
  const float wband = a.nbands == 2 ? 0.5f : 1.0f;
  float s[4][U];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int u = 0; u < U; ++u) s[v][u] = 0.f;
  for (int c0 = 0; c0 < nchan; c0 += CW) {
    // every load of the batch from a clamped slot first, then -inf past the candidates
    float z[CW][4][U];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int u = 0; u < U; ++u)
          z[cc][v][u] = zrow[(int64_t)min(c0 + cc, nchan - 1) * NBp + min(64 * v + lane + 256 * u, nC - 1)];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (64 * v + lane + 256 * u >= nC) z[cc][v][u] = -INFINITY;
    // Every channel of the batch is reduced (a channel past the last one only has its
    // result discarded): a branch here would let the compiler sink the later channels' loads
    // below it.  The maxima of all channels go through one interleaved reduction (a max is
    // exact in any order), then the lane sums of all channels through another.
    float mx[CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      mx[cc] = z[cc][0][0];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int u = 0; u < U; ++u) mx[cc] = fmaxf(mx[cc], z[cc][v][u]);
    }
    wave_max_dpp_n<CW>(mx);
    float sm[CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      float t[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        t[v] = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          z[cc][v][u] = fast_exp2(z[cc][v][u] - mx[cc]);   // -inf (not a candidate) -> 0
          t[v] += z[cc][v][u];
        }
      }
      sm[cc] = ((t[0] + t[1]) + t[2]) + t[3];
    }
    wave_sum_dpp_n<CW>(sm);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      const bool cv = c0 + cc < nchan;                 // uniform
      const float inv = wband / sm[cc];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float t = fmaf(z[cc][v][u], inv, s[v][u]);
          s[v][u] = cv ? t : s[v][u];
        }
    }
  }
  // keys in block order (free candidates only; scores are >= 0, so float bits order like values)
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = 64 * v + lane + 256 * u;
      keys[j] = (j < nC && j >= rp.nf_first && j < rp.last_lo) ? __float_as_uint(s[v][u]) + 1u : 0u;
    }
  wave_sync_lds();
  uint32_t k[KPL];
#pragma unroll
  for (int i = 0; i < KPL; i += 4) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(keys + KPL * lane + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) k[i + e] = t[e];
  }
  uint64_t flags = wave_topk<KPL>(k, rp.kp, rp.n_free, cand);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = KPL * lane + i;
    if (j < nC && (j < rp.nf_first || j >= rp.last_lo)) flags |= 1ull << i;    // forced blocks
  }
  wave_sync_lds();                                   // keys may be rewritten by the wave's next row
  return flags;
}

}  // namespace bsa
