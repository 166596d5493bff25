// Decode attention over the selected blocks, split over the KV list, and the
// fixed-order combine of split partials.
//
// Decode is memory bound (NSA page, decode-speed section: the speed-up tracks
// the tokens read).  Work is spread so that every CU streams a slice of the
// selected KV: one workgroup per (slice of the list, query row, KV group).  The
// G query heads of the group share each K/V load (NSA implementation-challenges
// section: GQA-aware access).  A thread's K and V loads are issued before any
// arithmetic.  Each workgroup writes an unnormalised partial (m, l, acc) per
// query head; the partials are merged in ascending slice order, so the result
// does not depend on scheduling.  The merge runs in the same launch: partials go
// out with device-scope stores and the workgroup that finishes a (row, group)'s
// last slice merges them (a kernel boundary costs more than the counter and the
// device-scope loads).  Past the counters' 1024 (batch, group, row) triples a
// combine kernel merges them instead, with the same arithmetic.
#include "common.h"
#include "internal.h"
#include "split.h"
#include "split_merge.h"
#include "dec_chunk.h"

namespace bsa {

// NSUB sub-chunks of kDecTok tokens form one chunk: the chunk's block indices
// are requested together, then all of its K/V rows, then the sub-chunks are
// computed in order (the same arithmetic as one sub-chunk at a time).
template <int DT, int D, int G, bool MERGE, int NSUB>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs a) {
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int LPT = D / 8;            // lanes per token
  constexpr int TPP = 64 / LPT;         // tokens per wave pass
  constexpr int TPW = kDecTok / 4;      // tokens per wave and sub-chunk
  constexpr int PASSES = TPW / TPP;     // passes per sub-chunk
  constexpr int NP = PASSES * NSUB;     // passes per chunk
  constexpr int CT = kDecTok * NSUB;    // tokens per chunk
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_acc[4][G][D];
  __shared__ int last_sh;
  __shared__ __attribute__((aligned(16))) uint64_t ml_sh[G * 32];   // the merge's (m, l): [head][slice of the batch]

  const int item = blockIdx.x, qb = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int tg = lane / LPT, d0 = (lane % LPT) * 8;
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  const int row = qb;                                   // one query row per block

  const int64_t t_begin = (int64_t)item * a.tok_per_item;
  const int qpos = a.q_pos0 + row;
  // The list count, the queries and the block indices of the first chunk are
  // loaded together: an index slot past the count holds a stale value that is
  // only used once the count has ruled it in.
  const int64_t cap_tok = (int64_t)a.cap * a.kv_block;
  int blk[NP], off[NP];
  // token of pass q (sub-chunk q / PASSES) of the chunk at c0 held by this lane
  auto tok = [&](int64_t c0, int q) __attribute__((always_inline)) {
    return c0 + (q / PASSES) * kDecTok + w * TPW + (q % PASSES) * TPP + tg;
  };
  auto load_blocks = [&](int64_t c0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t t = tok(c0, p);
      // 32-bit: list tokens stay below 2^31 (checked on the host)
      const int e = (int)((uint32_t)t / (uint32_t)a.kv_block);
      off[p] = (int)t - e * a.kv_block;
      blk[p] = t < cap_tok ? a.idx[li * a.cap + e] : -1;
    }
  };
  const int n_list = a.cnt[li];
  load_blocks(t_begin);
  // a stable row (mask 0) is skipped; its byte is read once the list's loads are out
  if (a.row_mask && a.row_mask[(int64_t)b * a.Lq + row] == 0) return;

  float qx[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load8<DT>(a.q + ((int64_t)b * a.qsb + (int64_t)(g * G + h) * a.qsh + (int64_t)row * a.qsl + d0) * ES, qx[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qx[h][e] *= a.c2;
  }
  const int64_t ntok = (int64_t)n_list * a.kv_block;
  // With a sliding window (NSA structure section), the items after the list's
  // own walk the row's window instead: the a.win keys ending at the row's
  // position, key = key0 + t.  The merge takes the two runs of items apart.
  int64_t t_lo = t_begin, t_end, key0 = -1;
  const int sel_items = (int)((ntok + a.tok_per_item - 1) / a.tok_per_item);
  if (a.win > 0 && item >= sel_items) {
    const int64_t hi = min((int64_t)a.L, (int64_t)qpos + 1), lo = max((int64_t)0, hi - a.win);
    t_lo = (int64_t)(item - sel_items) * a.tok_per_item;
    if (t_lo >= hi - lo) return;                        // past the window
    t_end = min(hi - lo, t_lo + a.tok_per_item);
    key0 = lo;
  } else {
    if (MERGE && ntok == 0 && item == 0) {              // nothing selected: O = 0, LSE = -inf
      const int Hq = a.Hkv * G;
      for (int i = tid; i < G * D; i += 256) {
        const int h = i / D, d = i - h * D;
        const int64_t oi = (int64_t)b * a.osb + (int64_t)(g * G + h) * a.osh + (int64_t)row * a.osl + d;
        if (a.o_f32) static_cast<float*>(a.o)[oi] = 0.f;
        else static_cast<uint16_t*>(a.o)[oi] = 0;
        if (d == 0) a.lse[((int64_t)b * Hq + g * G + h) * a.Lq + row] = -INFINITY;
      }
    }
    if (ntok == 0) return;                              // (split path: the combine writes O = 0, LSE = -inf)
    if (t_begin >= ntok) return;                        // no slice of the list for this workgroup
    t_end = min(ntok, t_begin + a.tok_per_item);
  }
  float wm[G], wl[G], wacc[G][8];                       // this wave's running state
#pragma unroll
  for (int h = 0; h < G; ++h) {
    wm[h] = -INFINITY;
    wl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) wacc[h][e] = 0.f;
  }
  const int gk = g / a.kv_div;                          // the K/V head of this list
  const uint8_t* kb = a.k + ((int64_t)b * a.ksb + (int64_t)gk * a.ksh + d0) * ES;
  const uint8_t* vb = a.v + ((int64_t)b * a.vsb + (int64_t)gk * a.vsh + d0) * ES;

  for (int64_t c0 = t_lo; c0 < t_end; c0 += CT) {
    if (c0 != t_begin && key0 < 0) load_blocks(c0);
    int pos[NP];
    bool ok[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t t = tok(c0, p);
      const int64_t key = key0 >= 0 ? key0 + t : (int64_t)blk[p] * a.kv_block + off[p];
      ok[p] = t < t_end && (key0 >= 0 || blk[p] >= 0) && key < a.L && (!a.causal || key <= qpos);
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
  __syncthreads();
  // merge the 4 waves into this workgroup's partial
  const int64_t pbase = (li * a.items + item) * G;
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
    if (MERGE) {
      st_dev(a.part_o + (pbase + h) * D + d, o);
      if (d == 0) st_dev2(a.part_ml + (pbase + h) * 2, M, lsum);
    } else {
      a.part_o[(pbase + h) * D + d] = o;
      if (d == 0) {
        a.part_ml[(pbase + h) * 2] = M;
        a.part_ml[(pbase + h) * 2 + 1] = lsum;
      }
    }
  }
  if (!MERGE) return;
  // every workgroup past this point holds one slice: one of the list's sel_items, or with a
  // window one of its n_win after them (the others returned)
  int n_win = 0;
  if (a.win > 0) {
    const int64_t hi = min((int64_t)a.L, (int64_t)qpos + 1), lo = max((int64_t)0, hi - a.win);
    n_win = (int)((hi - lo + a.tok_per_item - 1) / a.tok_per_item);
  }
  if (!arrive_last(a.arrivals + li * kArrivalStride, sel_items + n_win, last_sh)) return;
  const int Hq = a.Hkv * G;
  const float* po = a.part_o + li * a.items * G * D;
  const float* pml = a.part_ml + li * a.items * G * 2;
  const int64_t o_off = (int64_t)b * a.osb + (int64_t)(g * G) * a.osh + (int64_t)row * a.osl;
  const int64_t r0 = ((int64_t)b * Hq + g * G) * a.Lq + row;     // head g G's (row) entry
  if (a.win == 0) {
    merge_published<G, D>(po, pml, sel_items, ml_sh, a.o, a.o_f32, o_off, a.osh, a.lse + r0, a.Lq);
  } else {
    merge_published_window<G, D>(po, pml, sel_items, n_win, ml_sh, a.o, a.o_f32, o_off, a.osh, a.lse + 2 * r0,
                                 2 * (int64_t)a.Lq, a.gates ? a.gates + 2 * r0 : nullptr, 2 * (int64_t)a.Lq);
  }
}

// Decode attention for bf16 lists with D = 128 (and their sliding windows):
// the same slices, partials and merge as decode_kernel, with the vector work
// per token cut.  Per chunk of 128 list tokens each wave takes 32 keys:
//  * scores on the matrix cores: S^T (16 keys x 16 query columns) = K Q^T with
//    v_mfma_f32_16x16x32_bf16, K rows straight from HBM into the A operand,
//    the G query heads as columns (zero past G); a lane then holds 4 keys of
//    one head, and the head's max and sum over the wave's keys take two
//    cross-row exchanges instead of a 16-lane reduction per (token, head);
//  * p goes through LDS to the P V layout, where a lane holds 8 dims of every
//    fourth token (16-byte V loads) and accumulates over its tokens with no
//    exchange; the four token sets are summed once per slice.
// The scores are bf16 products summed in fp32 on the matrix core, then scaled
// by scale * log2 e (decode_kernel scales q first); both are within the
// rounding of fp32 accumulation of the same products.
// Chunks of 32 NWAVE tokens, 32 per working wave: NWAVE = 4 on lengthened
// slices; NWAVE = 2 on a single row's 64-token slices, NWAVE = 1 on 32-token
// slices (the other waves only join the workgroup's merge).
template <int G, bool MERGE, int NWAVE, bool WIN>
__global__ __launch_bounds__(256) void decode_wide_kernel(DecArgs a) {
  constexpr int D = 128;
  constexpr int CT = 32 * NWAVE;                   // tokens per chunk: 32 per working wave
  constexpr int GP = G < 4 ? 4 : G;                // p row stride (16-byte reads)
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_acc[4][G][D];
  __shared__ int last_sh;
  __shared__ __attribute__((aligned(16))) uint64_t ml_sh[G * 32];   // the merge's (m, l): [head][slice of the batch]
  __shared__ __attribute__((aligned(16))) float p_sh[4][32][GP];   // per wave: p of its 32 keys, per head
  __shared__ float al_sh[4][G];                                     // per wave: the chunk's rescale per head

  const int item = blockIdx.x, row = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;       // scores: key / head column, key quad; P V: dim group, token set
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + row;
  const int64_t t_begin = (int64_t)item * a.tok_per_item;
  const int qpos = a.q_pos0 + row;
  const int n_list = min(a.cnt[li], a.cap);             // (a count past the capacity reads no further)
  // Q^T operand: column = head (columns past G load a valid row, then zeroed), k = dims 32 ks + 8 kq + 0..7
  const int hq = g * G + min(col, G - 1);
  u32x4 qw[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qw[ks] = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.qsb + (int64_t)hq * a.qsh + (int64_t)row * a.qsl +
                                                    32 * ks + 8 * kq) * 2);
  if (a.row_mask && a.row_mask[(int64_t)b * a.Lq + row] == 0) return;   // a stable row is skipped
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, col < G ? qw[ks] : u32x4{0u, 0u, 0u, 0u});
  const int64_t ntok = (int64_t)n_list * a.kv_block;
  if (MERGE && !WIN && ntok == 0 && item == 0) {       // nothing selected: O = 0, LSE = -inf
    const int Hq = a.Hkv * G;
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, d = i - h * D;
      const int64_t oi = (int64_t)b * a.osb + (int64_t)(g * G + h) * a.osh + (int64_t)row * a.osl + d;
      if (a.o_f32) static_cast<float*>(a.o)[oi] = 0.f;
      else static_cast<uint16_t*>(a.o)[oi] = 0;
      if (d == 0) a.lse[((int64_t)b * Hq + g * G + h) * a.Lq + row] = -INFINITY;
    }
  }
  // With a sliding window (NSA structure section) the items after the list's walk the row's
  // window: the a.win keys ending at the row's position, key = key0 + t.
  const int sel_items = (int)((ntok + a.tok_per_item - 1) / a.tok_per_item);
  int64_t t_lo = t_begin, t_end, key0 = -1;
  if (WIN && item >= sel_items) {
    const int64_t hi = min((int64_t)a.L, (int64_t)qpos + 1), lo = max((int64_t)0, hi - a.win);
    t_lo = (int64_t)(item - sel_items) * a.tok_per_item;
    if (t_lo >= hi - lo) return;                        // past the window
    t_end = min(hi - lo, t_lo + a.tok_per_item);
    key0 = lo;
  } else {
    if (ntok == 0 || t_begin >= ntok) return;
    t_end = min(ntok, t_begin + a.tok_per_item);
  }
  const uint8_t* kb = a.k + ((int64_t)b * a.ksb + (int64_t)g * a.ksh) * 2;
  const uint8_t* vb = a.v + ((int64_t)b * a.vsb + (int64_t)g * a.vsh) * 2;
  const int32_t* lst = a.idx + li * a.cap;

  float m_run = -INFINITY, l_run = 0.f;                 // scores layout: head col
  float acc[G][8];                                      // P V layout: head h, dims 8 col + e, tokens = kq (mod 4)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // Per chunk a lane needs 10 list tokens: its K row in each 16-key half (key col) and its 8 V rows
  // (tokens 4 rd + kq).  A token is clamped into the slice so that every index load is valid (no
  // load under a branch); ok rules it out afterwards.  32-bit: list tokens < 2^30.
  // A chunk's list entries are requested while the previous chunk is computed, so each chunk
  // waits for one memory round trip (its K/V rows).
  auto fetch_idx = [&](int64_t c0, int (&bl)[10]) __attribute__((always_inline)) {
    const int64_t tw = c0 + 32 * w;
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int64_t t = j < 2 ? tw + 16 * j + col : tw + 4 * (j - 2) + kq;
      const int tc = (int)min(t, t_end - 1);
      const int e = (int)((uint32_t)tc / (uint32_t)a.kv_block);
      bl[j] = lst[WIN ? min(e, a.cap - 1) : e];        // (window items: unused, kept in the list)
    }
  };
  struct Rows {
    bf16x8 kf[2][4];
    u32x4 vr[8];
    bool kok[2], vok[8];
  };
  auto issue = [&](int64_t c0, const int (&bl)[10], Rows& R) __attribute__((always_inline)) {
    const int64_t tw = c0 + 32 * w;
    int pos[10];
    bool ok[10];
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int64_t t = j < 2 ? tw + 16 * j + col : tw + 4 * (j - 2) + kq;
      const int tc = (int)min(t, t_end - 1);
      const int e = (int)((uint32_t)tc / (uint32_t)a.kv_block);
      const bool wk = WIN && key0 >= 0;               // a window item: contiguous keys
      const int64_t key = wk ? key0 + t : (int64_t)bl[j] * a.kv_block + (tc - e * a.kv_block);
      ok[j] = t < t_end && (wk || bl[j] >= 0) && key < a.L && (!a.causal || key <= qpos);
      pos[j] = ok[j] ? (int)key : 0;
    }
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      R.kok[kg] = ok[kg];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        R.kf[kg][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(kb + ((int64_t)pos[kg] * a.ksl + 32 * ks + 8 * kq) * 2));
    }
#pragma unroll
    for (int rd = 0; rd < 8; ++rd) {
      R.vok[rd] = ok[2 + rd];
      R.vr[rd] = *reinterpret_cast<const u32x4*>(vb + ((int64_t)pos[2 + rd] * a.vsl + 8 * col) * 2);
    }
  };
  if (w < NWAVE) {                                      // (wave-uniform)
    int bl[10];
    Rows R;
    fetch_idx(t_lo, bl);
    for (int64_t c0 = t_lo; c0 < t_end; c0 += CT) {
      issue(c0, bl, R);
      if (c0 + CT < t_end) fetch_idx(c0 + CT, bl);      // uniform; arrives while this chunk is computed
      dec_wide_chunk<G>(qb, R.kf, R.vr, R.kok, R.vok, a.c2, m_run, l_run, acc, p_sh[w], al_sh[w]);
    }
  }
  // the four token sets summed (the same bits on every row); row 0 of the wave holds the result
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
  __syncthreads();
  // merge the 4 waves into this workgroup's partial
  const int64_t pbase = (li * a.items + item) * G;
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
    if (MERGE) {
      st_dev(a.part_o + (pbase + h) * D + d, o);
      if (d == 0) st_dev2(a.part_ml + (pbase + h) * 2, M, lsum);
    } else {
      a.part_o[(pbase + h) * D + d] = o;
      if (d == 0) {
        a.part_ml[(pbase + h) * 2] = M;
        a.part_ml[(pbase + h) * 2 + 1] = lsum;
      }
    }
  }
  if (!MERGE) return;
  int n_win = 0;
  if constexpr (WIN) {
    const int64_t hi = min((int64_t)a.L, (int64_t)qpos + 1), lo = max((int64_t)0, hi - a.win);
    n_win = (int)((hi - lo + a.tok_per_item - 1) / a.tok_per_item);
  }
  if (!arrive_last(a.arrivals + li * kArrivalStride, sel_items + n_win, last_sh)) return;
  const int Hq = a.Hkv * G;
  const float* po = a.part_o + li * a.items * G * D;
  const float* pml = a.part_ml + li * a.items * G * 2;
  const int64_t o_off = (int64_t)b * a.osb + (int64_t)(g * G) * a.osh + (int64_t)row * a.osl;
  const int64_t r0 = ((int64_t)b * Hq + g * G) * a.Lq + row;     // head g G's (row) entry
  if constexpr (!WIN) {
    merge_published<G, D>(po, pml, sel_items, ml_sh, a.o, a.o_f32, o_off, a.osh, a.lse + r0, a.Lq);
  } else {
    merge_published_window<G, D>(po, pml, sel_items, n_win, ml_sh, a.o, a.o_f32, o_off, a.osh, a.lse + 2 * r0,
                                 2 * (int64_t)a.Lq, a.gates ? a.gates + 2 * r0 : nullptr, 2 * (int64_t)a.Lq);
  }
}

// Merge the split partials of active (row, head) pairs of a query block in
// ascending slice order; write O (q's dtype) and the natural-log LSE.  One
// thread per (query vector, dim).  Per batch of BATCH slices, the (m, l) pairs
// of the workgroup's query vectors go through LDS (one load per thread) while
// each thread loads its dim of every partial O, so a thread has at most
// BATCH + 1 loads in flight and none waits for a free counter slot; the merge
// then runs with a running maximum, BATCH slices at a time.
template <int ODT, int BATCH>
__global__ __launch_bounds__(256) void combine_kernel(CombArgs a) {
  __shared__ __attribute__((aligned(16))) uint64_t ml_sh[2][4 * BATCH];   // [parity][query vector][slice]
  const int QVC = a.qvc;                           // 256 / D <= 4
  const int nchunk = (a.QV + QVC - 1) / QVC;
  const int qb = blockIdx.x / nchunk, qv0 = (blockIdx.x % nchunk) * QVC;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, QV = a.QV, D = a.D, Hq = a.Hkv * G;
  const int tid = threadIdx.x;
  const int c = tid / D, d = tid - c * D;          // 256 threads cover QVC * D <= 256 (D >= 64)
  const int qv = qv0 + c;
  const int rl = qv / G, hl = qv - rl * G;
  const int row = qb * a.q_block + rl;
  // every thread takes part in the barriers; only live ones write.  The row-mask byte is loaded
  // for a valid row whatever this thread's (no load under a branch) and looked at after the batch
  const uint8_t* rmp = a.row_mask ? a.row_mask + (int64_t)b * a.Lq + min(row, a.Lq - 1)
                                  : reinterpret_cast<const uint8_t*>(a.part_ml);   // any readable byte
  const uint8_t rbyte = *rmp;
  const bool in_range = c < QVC && qv < QV && row < a.Lq;
  // a workgroup whose rows are all stable has no partials to merge (none were written): it leaves
  // before requesting any, rather than pulling unwritten slots from memory
  if (a.row_mask && !__syncthreads_or(in_range && rbyte != 0)) return;
  bool live = false;                               // set once the first batch is requested
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  const int64_t p0 = li * a.items;
  // Slots are clamped to the workspace, not to the valid count, so the first
  // batch loads together with the count; slots past the count may hold stale
  // values and are excluded by selects (never multiplied by a zero weight).
  const int qvo = min(qv, QV - 1);                 // a dead thread loads a valid slot too: no load under a branch
  const uint32_t lo_o = (uint32_t)(qvo * D + d);
  const int cs = tid / BATCH, us = tid - cs * BATCH;   // the (m, l) this thread stages: query vector qv0 + cs, slice us
  const uint32_t lo_ml = (uint32_t)min(qv0 + cs, QV - 1) * 2u;
  auto issue = [&](int it0, uint64_t& mlv, float (&ov)[BATCH]) __attribute__((always_inline)) {
    mlv = 0;
    if (tid < QVC * BATCH) {
      const int64_t it = min(it0 + us, a.items - 1);
      mlv = *reinterpret_cast<const uint64_t*>(a.part_ml + (p0 + it) * QV * 2 + lo_ml);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t it = min(it0 + u, a.items - 1);
      ov[u] = a.part_o[(p0 + it) * QV * D + lo_o];
    }
  };
  int parity = 0;
  // merge items [first, first + n) in order; the batch at `first` is issued already
  auto merge = [&](int first, int n, uint64_t mlv, float (&ov)[BATCH], float& M, float& L, float& acc)
      __attribute__((always_inline)) {
    M = -INFINITY;
    L = 0.f;
    acc = 0.f;
    for (int it0 = 0; it0 < n; it0 += BATCH) {     // n is uniform over the workgroup
      if (it0 > 0) issue(first + it0, mlv, ov);
      if (tid < QVC * BATCH) ml_sh[parity][tid] = mlv;
      __syncthreads();
      if (live) {
        uint64_t mlr[BATCH];
#pragma unroll
        for (int q = 0; q < BATCH / 2; ++q) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(&ml_sh[parity][c * BATCH + 2 * q]);
          mlr[2 * q] = (uint64_t)t[0] | ((uint64_t)t[1] << 32);
          mlr[2 * q + 1] = (uint64_t)t[2] | ((uint64_t)t[3] << 32);
        }
        float bm = M;
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (it0 + u < n) bm = fmaxf(bm, __uint_as_float((uint32_t)mlr[u]));
        if (bm != -INFINITY) {                     // else nothing visible so far
          const float alpha = M == -INFINITY ? 0.f : fast_exp2(M - bm);
          L *= alpha;
          acc *= alpha;
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const float mv = __uint_as_float((uint32_t)mlr[u]);
            // selects, not a branch per slice (a skipped slot's stale values are never multiplied in)
            const bool use = it0 + u < n && mv != -INFINITY;
            const float wgt = fast_exp2(mv - bm);
            const float l2 = fmaf(__uint_as_float((uint32_t)(mlr[u] >> 32)), wgt, L), a2 = fmaf(ov[u], wgt, acc);
            L = use ? l2 : L;
            acc = use ? a2 : acc;
          }
          M = bm;
        }
      }
      parity ^= 1;                                 // the next batch writes the other buffer
    }
  };
  uint64_t mlv;
  float ov[BATCH];
  issue(0, mlv, ov);
  live = in_range && !(a.row_mask && rbyte == 0);
  int nvalid;
  if (a.per_item_from_count) {
    const int c_list = a.cnt[li];
    const int per = split_per(c_list, a.items);
    nvalid = (c_list + per - 1) / per;
  } else {
    const int64_t nunits = a.cnt ? (int64_t)a.cnt[li] * a.unit_num : (int64_t)a.items * a.unit_den;
    nvalid = (int)min((int64_t)a.items, (nunits + a.unit_den - 1) / a.unit_den);
  }
  float M, L, acc;
  merge(0, nvalid, mlv, ov, M, L, acc);
  const int h = g * G + hl;
  const int64_t oi = (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)row * a.osl + d;
  float out = L > 0.f ? acc / L : 0.f;
  if (a.win > 0) {
    // the window's items follow the list's: O = g_sel O_sel + g_win O_win, one LSE per branch
    // (decode only: one row per query block, so the window is uniform over the workgroup)
    const int64_t qpos = (int64_t)a.q_pos0 + qb * a.q_block;
    const int64_t hi = min((int64_t)a.L, qpos + 1), nwin = hi - max((int64_t)0, hi - a.win);
    const int nw = (int)((nwin + a.unit_den - 1) / a.unit_den);
    issue(nvalid, mlv, ov);
    float Mw, Lw, accw;
    merge(nvalid, nw, mlv, ov, Mw, Lw, accw);
    if (live) {
      const int64_t gi = (((int64_t)b * Hq + h) * a.Lq + row) * 2;
      const float g0 = a.gates ? a.gates[gi] : 1.f, g1 = a.gates ? a.gates[gi + 1] : 1.f;
      out = g0 * out + g1 * (Lw > 0.f ? accw / Lw : 0.f);
      if (d == 0) {
        a.lse[gi] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
        a.lse[gi + 1] = Lw > 0.f ? (Mw + log2f(Lw)) * kLn2 : -INFINITY;
      }
    }
  } else if (live && d == 0) {
    a.lse[((int64_t)b * Hq + h) * a.Lq + row] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  if (!live) return;
  if (ODT == BSA_BF16) reinterpret_cast<uint16_t*>(a.o)[oi] = (uint16_t)f32_to_bf16(out);
  else reinterpret_cast<float*>(a.o)[oi] = out;
}

// Batches of 32: the first batch is loaded whatever the valid count (so it
// goes out with the count), and split lists are usually far shorter than
// their capacity, so a wider first batch mostly loads unused slots (measured
// on the denoising step: 6.3 us at 32, 14.9 us at 64).
void launch_combine(const CombArgs& a, int odt, int B, hipStream_t s) {
  dim3 grid(a.NQB * ((a.QV + a.qvc - 1) / a.qvc), a.Hkv, B);
  if (odt == BSA_BF16) hipLaunchKernelGGL((combine_kernel<BSA_BF16, 32>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((combine_kernel<BSA_F32, 32>), grid, dim3(256), 0, s, a);
}

void launch_decode(const DecArgs& a, int dt, int D, int G, int B, hipStream_t s) {
  dim3 grid(a.items, a.NQB, B * a.Hkv);
  const bool wide = a.tok_per_item % (kDecTok * kDecWideSub) == 0;
  if (dt == BSA_BF16 && D == 128 && a.kv_div == 1) {
    // bf16 lists with D = 128 (and their windows): the matrix-core form, on all four waves for
    // lengthened slices
#define BSA_DECW_W(GG, WW)                                                                                   \
  do {                                                                                                       \
    if (wide) {                                                                                              \
      if (a.arrivals) hipLaunchKernelGGL((decode_wide_kernel<GG, true, 4, WW>), grid, dim3(256), 0, s, a);   \
      else hipLaunchKernelGGL((decode_wide_kernel<GG, false, 4, WW>), grid, dim3(256), 0, s, a);             \
    } else if (a.tok_per_item % 64 == 0) {                                                                   \
      if (a.arrivals) hipLaunchKernelGGL((decode_wide_kernel<GG, true, 2, WW>), grid, dim3(256), 0, s, a);   \
      else hipLaunchKernelGGL((decode_wide_kernel<GG, false, 2, WW>), grid, dim3(256), 0, s, a);             \
    } else {                                                                                                 \
      if (a.arrivals) hipLaunchKernelGGL((decode_wide_kernel<GG, true, 1, WW>), grid, dim3(256), 0, s, a);   \
      else hipLaunchKernelGGL((decode_wide_kernel<GG, false, 1, WW>), grid, dim3(256), 0, s, a);             \
    }                                                                                                        \
  } while (0)
#define BSA_DECW(GG)                                                                                         \
  do {                                                                                                       \
    if (a.win > 0) BSA_DECW_W(GG, true); else BSA_DECW_W(GG, false);                                        \
  } while (0)
    switch (G) {
      case 1: BSA_DECW(1); break;
      case 2: BSA_DECW(2); break;
      case 4: BSA_DECW(4); break;
      default: BSA_DECW(8); break;
    }
#undef BSA_DECW
#undef BSA_DECW_W
    return;
  }
#define BSA_DEC(DT, DD, GG)                                                                                     \
  do {                                                                                                          \
    if (wide) {                                                                                                 \
      if (a.arrivals) hipLaunchKernelGGL((decode_kernel<DT, DD, GG, true, kDecWideSub>), grid, dim3(256), 0, s, a); \
      else hipLaunchKernelGGL((decode_kernel<DT, DD, GG, false, kDecWideSub>), grid, dim3(256), 0, s, a);        \
    } else {                                                                                                    \
      if (a.arrivals) hipLaunchKernelGGL((decode_kernel<DT, DD, GG, true, 1>), grid, dim3(256), 0, s, a);       \
      else hipLaunchKernelGGL((decode_kernel<DT, DD, GG, false, 1>), grid, dim3(256), 0, s, a);                 \
    }                                                                                                           \
  } while (0)
#define BSA_DEC_G(DT, DD)                              \
  do {                                                 \
    switch (G) {                                       \
      case 1: BSA_DEC(DT, DD, 1); break;               \
      case 2: BSA_DEC(DT, DD, 2); break;               \
      case 4: BSA_DEC(DT, DD, 4); break;               \
      default: BSA_DEC(DT, DD, 8); break;              \
    }                                                  \
  } while (0)
  if (dt == BSA_BF16) {
    if (D == 128) BSA_DEC_G(BSA_BF16, 128); else BSA_DEC_G(BSA_BF16, 64);
  } else {
    if (D == 128) BSA_DEC_G(BSA_F32, 128); else BSA_DEC_G(BSA_F32, 64);
  }
#undef BSA_DEC_G
#undef BSA_DEC
}

}  // namespace bsa
