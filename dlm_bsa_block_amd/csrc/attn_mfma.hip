// Gather-by-block-index attention with bf16 MFMA tiles (FASA page sec. 2:
// full head-dim attention over only the selected tokens, at their original
// positions).  Used for
//   * causal sparse prefill: one workgroup per (query block of 128 rows, query
//     head) walking the group's list of KV tiles; workgroups that share a KV
//     group are placed on the same XCD, heads of one query block next to each
//     other, so their K/V tiles are re-read from that XCD's L2;
//   * the denoising step: one workgroup per (slice of the list, query block,
//     KV group) holding the block's active (row, head) pairs as up to 128
//     query vectors, writing split partials for the combine (LoSA sec. 2:
//     only active rows recompute, over the block's union).  In the fused
//     denoising step the workgroup first picks the blocks of every active
//     row itself (one wavefront per row, from the logits) and takes the
//     union, so no launch sits between the logits and the attention.
// K/V tiles are copied straight from global memory into LDS (double-buffered)
// and shared by the waves of a workgroup; each wave owns 32 query vectors.
// Online softmax in fp32 with exp2; the running max and sum are lane-local
// (see mfma_tile.h).
#include <algorithm>

#include "internal.h"
#include "mfma_tile.h"
#include "pick.h"
#include "split.h"
#include "split_merge.h"

namespace bsa {

struct GatherArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl;
  const int32_t* idx;
  const int32_t* cnt;
  int B, cap, NQB, Hkv, G, L, Lq, q_block, q_pos0, causal;
  float c2;                       // scale * log2(e)
  const uint8_t* row_mask;
  void* o;                        // bf16, or f32 when o_f32
  int o_f32;
  int64_t osb, osh, osl;
  float* lse;
  float* part_o;
  float* part_ml;
  int items;
  int wpg;                        // streaming kernel: workgroups per (batch, KV group)
  PickArgs pk;                    // in-kernel pick (split mode, one query block): Z, row plan inputs
};

// One workgroup = NW waves of 32 query vectors.  Direct mode: NW / 4 heads of
// one KV group (4 waves of 32 rows each per head) share every K/V tile.  Split
// mode (NW = 4): the active (row, head) pairs of a query block, compacted.
// K/V tiles are double-buffered in LDS: the copy of tile u + 1 runs while
// tile u is computed, so one barrier per tile suffices.  A list entry (a KV
// block of SUB * KVB keys) is walked as SUB tiles of KVB keys: with 64-key
// tiles two workgroups fit on a CU and their waves overlap freely.
// PU > 0 (split mode, one query block): the list is not read but picked here
// -- wavefront w picks active rows w, w + NW, ... (wave_pick_row<PU>, the
// keys staged in the tile buffers, which are free until the walk starts), the
// flags are OR-ed over the waves and compacted; every workgroup of the group
// computes the same list, keeps its own slice of it in LDS, and workgroup 0
// writes the list and its length out.
template <int KVB, int NW, bool SPLIT, int SUB = 1, int PU = 0>
__global__ __launch_bounds__(NW * 64, (NW == 4 && KVB == 64) ? 2 : 1) void gather_mfma_kernel(GatherArgs a) {
  constexpr int TILE = KVB * kRow;                 // elements of one K or V tile
  constexpr int HPW = SPLIT ? 1 : NW / 4;          // heads per workgroup
  constexpr bool PICK = PU > 0;
  static_assert(!PICK || (SPLIT && 256 * PU * NW * 4 <= 4 * TILE * 2), "pick keys fit in the tile buffers");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE];   // K0 V0 K1 V1
  __shared__ int qv_row[128], qv_head[128], qv_full[128];
  __shared__ int n_qv_sh;
  __shared__ uint64_t pflags_sh[PICK ? NW : 1][64];
  __shared__ __attribute__((aligned(16))) uint32_t pcand_sh[PICK ? NW : 1][64];
  __shared__ int slice_sh[PICK ? kSplitBlocks : 1];
  __shared__ int n_list_sh;

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, g, qb, item = 0, h0 = 0;
  if (SPLIT) {
    item = blockIdx.x;
    qb = blockIdx.y;
    b = blockIdx.z / a.Hkv;
    g = blockIdx.z - b * a.Hkv;
  } else {
    // XCD-aware order: workgroup n runs on XCD n % 8; give each XCD a contiguous
    // run of (batch, group, query block descending, head set) work items.
    const int total = gridDim.x;
    const int n = blockIdx.x;
    const int i = (total % 8 == 0) ? (n % 8) * (total / 8) + n / 8 : n;
    const int sets = a.G / HPW;
    h0 = (i % sets) * HPW;
    const int rest = i / sets;
    qb = a.NQB - 1 - rest % a.NQB;
    const int bgi = rest / a.NQB;
    b = bgi / a.Hkv;
    g = bgi - b * a.Hkv;
  }
  const int64_t li = ((int64_t)b * a.Hkv + g) * a.NQB + qb;
  // query vectors of this workgroup
  auto stage_qv = [&]() __attribute__((always_inline)) {
    if (w == 0) {
      const int row = qb * a.q_block + lane;
      const bool act = lane < a.q_block && row < a.Lq && (!a.row_mask || a.row_mask[(int64_t)b * a.Lq + row]);
      const unsigned long long m = __ballot(act);
      if (act) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        for (int hh = 0; hh < a.G; ++hh) {
          qv_row[rank * a.G + hh] = row;
          qv_head[rank * a.G + hh] = hh;
          qv_full[rank * a.G + hh] = lane * a.G + hh;
        }
      }
      if (lane == 0) n_qv_sh = __popcll(m) * a.G;
    }
    __syncthreads();
  };
  // this lane's query vector and its fragments
  const int wr = w & 3;                            // wave within its head
  const int qv = 32 * wr + r32;
  int n_qv = 0, row = 0, h = 0;
  bool valid = false, wave_busy = false;
  bf16x8 qf[8];
  auto setup_q = [&]() __attribute__((always_inline)) {
    if (SPLIT) {
      n_qv = n_qv_sh;
      valid = qv < n_qv;
      row = valid ? qv_row[qv] : 0;
      h = g * a.G + (valid ? qv_head[qv] : 0);
    } else {
      row = qb * a.q_block + qv;
      valid = qv < a.q_block && row < a.Lq;
      h = g * a.G + h0 + (w >> 2);
    }
    wave_busy = SPLIT ? (32 * wr < n_qv) : (32 * wr < a.q_block && qb * a.q_block + 32 * wr < a.Lq);
    // an invalid lane reads a row inside the sequence (row 0 in split mode, else the last row);
    // its fragments are zeroed where they are first needed, so nothing waits for the loads here
    load_q_frag_raw(a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)min(row, a.Lq - 1) * a.qsl, qf);
  };
  int n_list = 0, e0 = 0, e1;
  // requested before the row mask and the queries (a count above the capacity is cut to it)
  if constexpr (!PICK) n_list = min(a.cnt[li], a.cap);
  if constexpr (PICK) {
    stage_qv();
    setup_q();                                     // the query loads overlap the picks
    const int n_act = n_qv_sh / a.G;
    uint64_t fl = 0;
    uint32_t* keys = reinterpret_cast<uint32_t*>(lds) + w * 256 * PU;
    for (int k = w; k < n_act; k += NW) fl |= wave_pick_row<PU>(a.pk, b, g, qv_row[k * a.G], keys, pcand_sh[w]);
    pflags_sh[w][lane] = fl;
    __syncthreads();
    if (w == 0) {
      uint64_t f = pflags_sh[0][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) f |= pflags_sh[ww][lane];
      // ascending compaction (bit e of lane l = block 4 PU l + e); this workgroup keeps its slice
      const uint32_t c = (uint32_t)__popcll(f);
      const uint32_t incl = wave_incl_scan_dpp(c);
      const int n = (int)lane_read(incl, 63);
      const int per = split_per(n, a.items);
      const int s0 = item * per, s1 = min(n, s0 + per);
      int pos = (int)(incl - c);
      int32_t* out = a.pk.idx + li * a.cap;            // the pick writes the list (workgroup 0)
      while (f) {
        const int e = __ffsll((unsigned long long)f) - 1;
        f &= f - 1;
        const int j = 4 * PU * lane + e;
        if (pos >= s0 && pos < s1 && pos - s0 < kSplitBlocks) slice_sh[pos - s0] = j;   // per <= kSplitBlocks
        if (item == 0) out[pos] = j;
        ++pos;
      }
      if (lane == 0) {
        n_list_sh = n;
        if (item == 0) a.pk.cnt[li] = n;
      }
    }
    __syncthreads();
    n_list = n_list_sh;
  } else if (SPLIT) {
    // the active rows and their query loads do not depend on the list: both overlap its length's load
    stage_qv();
    setup_q();
  }
  e1 = n_list;
  if (SPLIT) {
    // the list's entries are shared out over the launched items: a short list (a
    // few active rows' union) gets one entry per workgroup, a full one kSplitBlocks
    const int per = split_per(n_list, a.items);
    e0 = item * per;
    if (e0 >= n_list) return;
    e1 = min(n_list, e0 + per);
  }
  if (!SPLIT) setup_q();
  zero_q_frag(valid, qf);
  const int qpos = a.q_pos0 + row;
  // smallest query position of the wave (for deciding whether a tile needs the causal mask)
  int wave_min_pos = valid ? qpos : 0x7FFFFFFF;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_min_pos = min(wave_min_pos, wave_xor(wave_min_pos, m));

  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  const int32_t* list = a.idx + li * a.cap;
  // a split slice's entries (at most kSplitBlocks), one per lane, read once: no list load inside the walk
  int ent = -1;
  if constexpr (SPLIT) {
    if constexpr (PICK) ent = lane < e1 - e0 ? slice_sh[lane] : -1;
    else ent = lane < e1 - e0 ? list[e0 + lane] : -1;
  }
  // rows of tile u (of list entry e0 + u / SUB) inside the KV sequence (0 for
  // an index outside it, or a part beyond the end: nothing is read)
  auto entry_rows = [&](int u, int& key0) {
    const int j = SPLIT ? __builtin_amdgcn_readlane(ent, u / SUB) : list[e0 + u / SUB];
    const int blk0 = j * (KVB * SUB);
    key0 = blk0 + (u % SUB) * KVB;
    return (j < 0 || blk0 >= a.L || key0 >= a.L) ? 0 : min(KVB, a.L - key0);
  };
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int e, int buf) {
    int key0;
    const int nk = entry_rows(e, key0);
    if (nk == 0) return;
    issue_tile<KVB, NW>(kbg + (int64_t)key0 * a.ksl, a.ksl, nk, lds0 + (uint32_t)(buf * 2 * TILE * 2));
    issue_tile<KVB, NW>(vbg + (int64_t)key0 * a.vsl, a.vsl, nk, lds0 + (uint32_t)((buf * 2 + 1) * TILE * 2));
  };


  const int nt = (e1 - e0) * SUB;
  // largest query position of the wave: a tile wholly after it is skipped
  int wave_max_pos = valid ? qpos : -1;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) wave_max_pos = max(wave_max_pos, wave_xor(wave_max_pos, m));
  wave_max_pos = __builtin_amdgcn_readfirstlane(wave_max_pos);
  if (nt > 0) issue(0, 0);
  for (int u = 0; u < nt; ++u) {
    const int buf = u & 1;
    int key0;
    const int nk = entry_rows(u, key0);
    wait_tile_loads();                             // this wave's part of tile u is in LDS
    __syncthreads();                               // ... and everyone's; tile u - 1 is finished
    if (u + 1 < nt) issue(u + 1, buf ^ 1);
    if (nk == 0 || !wave_busy || (a.causal && key0 > wave_max_pos)) continue;
    const uint16_t* Ks = lds + buf * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;
    f32x16 s[KVB / 32];
    qk_tile<KVB>(Ks, kofs, qf, s);
    const bool need_mask = nk < KVB || (a.causal && key0 + KVB - 1 > wave_min_pos);
    if (need_mask) {
      // largest visible key offset of this lane's query in the tile
      int lim = nk - 1;
      if (a.causal) lim = min(lim, qpos - key0);
      mask_tile<KVB / 32>(s, lim);
    }
    const float msub = softmax_rescale(tile_max<KVB / 32>(s) * a.c2, m_ref, l_run, o);
    softmax_pv_tile<KVB>(Vs, vofs, s, a.c2, msub, l_run, o);
  }

  if (!wave_busy) return;
  const float l_tot = pair_sum(l_run);
  if (!SPLIT) {
    if (!valid) return;
    if (a.row_mask && a.row_mask[(int64_t)b * a.Lq + row] == 0) return;   // stable row: cached O/LSE stay
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t oi = (int64_t)b * a.osb + (int64_t)h * a.osh + (int64_t)row * a.osl;
    store_o_row(a.o_f32 ? (void*)(static_cast<float*>(a.o) + oi) : (void*)(static_cast<uint16_t*>(a.o) + oi),
                a.o_f32, o, inv, lane >> 5);
    if (lane < 32)
      a.lse[((int64_t)b * a.Hkv * a.G + h) * a.Lq + row] =
          l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    if (!valid) return;
    const int QV = a.q_block * a.G;
    const int64_t pi = (li * a.items + item) * QV + qv_full[qv];
    float* po = a.part_o + pi * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = o_dim(dt, 4 * i4);
        f32x4 v4 = {o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(po + d) = v4;
      }
    if (lane < 32) {
      a.part_ml[pi * 2] = m_ref;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

// Direct mode for an even group size: one workgroup = 8 waves = two heads of
// one KV group over a query block of up to 128 rows (waves 0-3 head h0 =
// group A, waves 4-7 head h0 + 1 = group B).  Waves w and w + 4 share a SIMD,
// so the two groups run half a list entry apart: while A computes S = K Q^T
// of entry e on the matrix cores, B runs the softmax and P V of entry e - 1,
// and the other way round in the next phase.  The vector-ALU softmax of one
// wave then overlaps the MFMA work of its partner instead of queueing behind
// the barriers that keep the groups in step.  K and V have two LDS buffers
// each; the K copy of entry e + 1 is issued once B has finished reading the
// K buffer it replaces (one phase after A did), the V copy likewise, so each
// copy has a whole entry of compute to land.
//
// The work items of one (batch, KV group) -- (query block, head pair) -- are
// dealt out to wpg workgroups (about one per CU), largest query block first
// and in alternating direction per round, so every workgroup gets a
// near-equal share of tiles.  A workgroup stages the lists of all its items in
// LDS once and walks them as one stream of list entries: the copies, barriers
// and the half-entry offset of the two groups run on across item boundaries,
// so starting an item costs neither a list round trip nor a pipeline fill.
// An item's list is walked from its highest block down: the diagonal tile,
// whose nearby keys tend to score highest, comes first and sets a running
// max that later tiles seldom raise, which skips most O rescales (the sum is
// order-independent up to rounding).
// Workgroup n runs on XCD n % 8 and serves KV group n % (B * Hkv), so a
// group's K/V tiles stay in the L2 of its XCD.
constexpr int kMaxItemsWG = 64;    // work items one streaming workgroup takes

template <int KVB>
__global__ __launch_bounds__(512, 1) void gather_stream_kernel(GatherArgs a) {
  constexpr int NW = 8;
  constexpr int TILE = KVB * kRow;
  constexpr int IT = KVB / 4 / NW;                 // copy instructions per wave for one K or V tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * TILE];   // K0 K1 V0 V1
  __shared__ int list_sh[kMaxListMfma];
  __shared__ uint8_t ent_sh[kMaxListMfma];         // item | 64 (first entry of it) | 128 (last entry)
  __shared__ int it_r[kMaxItemsWG], it_start[kMaxItemsWG + 1];
  __shared__ uint32_t empty_sh[2];

  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wr = w & 3;
  const int BG = a.B * a.Hkv, bg = blockIdx.x % BG, slot = blockIdx.x / BG;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int sets = a.G / 2, NI = a.NQB * sets, S = a.wpg;
  // item i of this workgroup: rank r of the group's items (largest query block first)
  auto item_rank = [&](int i) __attribute__((always_inline)) {
    return i * S + ((i & 1) ? S - 1 - slot : slot);
  };
  const int rounds = (NI + S - 1) / S;
  const int nit = rounds == 0 ? 0 : rounds - 1 + (item_rank(rounds - 1) < NI ? 1 : 0);
  if (nit == 0) return;                            // uniform over the workgroup

  // Per-item state of a wave, all wave-uniform: the lane's query is row
  // wmin - q_pos0 + r32 of head h.
  struct Ctx {
    int h, wmin;
    bool busy;
  };
  auto ctx = [&](int r) __attribute__((always_inline)) {
    Ctx c;
    const int qb = a.NQB - 1 - r / sets;
    c.h = g * a.G + (r % sets) * 2 + grp;
    c.busy = 32 * wr < a.q_block && qb * a.q_block + 32 * wr < a.Lq;
    c.wmin = a.q_pos0 + qb * a.q_block + 32 * wr;  // smallest query position of the wave
    return c;
  };
  const int64_t li0 = (int64_t)bg * a.NQB;
  bf16x8 qf[8];
  // Per-lane address terms below come from a copy of threadIdx.x passed
  // through an empty asm, so they are rebuilt where used instead of being held
  // (and spilled) across the loop: a spill reload would wait for every tile
  // copy in flight.
  auto lane_id = []() __attribute__((always_inline)) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & 63;
  };
  auto load_q = [&](const Ctx& c) __attribute__((always_inline)) {
    const int ln = lane_id();
    const int row = c.wmin - a.q_pos0 + (ln & 31);
    const bool ok = 32 * wr + (ln & 31) < a.q_block && row < a.Lq;
    const uint16_t* qrow = a.q + (int64_t)b * a.qsb + (int64_t)c.h * a.qsh + (int64_t)row * a.qsl;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * (ln >> 5)) : u32x4{0, 0, 0, 0};
      qf[st] = __builtin_bit_cast(bf16x8, v);
    }
  };

  Ctx cur = ctx(item_rank(0));
  load_q(cur);
  // item table and the flattened list
  if (w == 0) {
    int n_i = 0;
    if (lane < nit) {
      const int r = item_rank(lane);
      n_i = min(a.cnt[li0 + (a.NQB - 1 - r / sets)], a.cap);
      it_r[lane] = r;
    }
    const int incl = (int)wave_incl_scan_dpp((uint32_t)n_i);
    if (lane < nit) it_start[lane + 1] = incl;
    if (lane == 0) it_start[0] = 0;
    const unsigned long long em = __ballot(lane < nit && n_i == 0);
    if (lane == 0) { empty_sh[0] = (uint32_t)em; empty_sh[1] = (uint32_t)(em >> 32); }
  }
  __syncthreads();
  const int N = __builtin_amdgcn_readfirstlane(it_start[nit]);
  for (int e = tid; e < N; e += NW * 64) {
    int lo = 0, hi = nit - 1;                      // the item whose entries hold e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (it_start[mid] <= e) lo = mid; else hi = mid - 1;
    }
    const int st = it_start[lo], n = it_start[lo + 1] - st;
    const int qb = a.NQB - 1 - it_r[lo] / sets;
    list_sh[e] = a.idx[(li0 + qb) * a.cap + (n - 1 - (e - st))];   // highest block first
    ent_sh[e] = (uint8_t)(lo | (e == st ? 64 : 0) | (e + 1 == it_start[lo + 1] ? 128 : 0));
  }
  __syncthreads();

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  auto epilogue = [&](const Ctx& c) __attribute__((always_inline)) {
    if (!c.busy) return;
    const float l_tot = pair_sum(l_run);
    const int ln = lane_id();
    const int row = c.wmin - a.q_pos0 + (ln & 31);
    if (32 * wr + (ln & 31) >= a.q_block || row >= a.Lq) return;
    // a stable row (row_mask 0) keeps its cached O/LSE; the load is made only when a mask is given
    if (a.row_mask && a.row_mask[(int64_t)b * a.Lq + row] == 0) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t oi = (int64_t)b * a.osb + (int64_t)c.h * a.osh + (int64_t)row * a.osl;
    store_o_row(a.o_f32 ? (void*)(static_cast<float*>(a.o) + oi) : (void*)(static_cast<uint16_t*>(a.o) + oi),
                a.o_f32, o, inv, ln >> 5);
    if (ln < 32)
      a.lse[((int64_t)b * a.Hkv * a.G + c.h) * a.Lq + row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  };
  // items with an empty list: O = 0, LSE = -inf (o, m, l hold exactly that now)
  {
    unsigned long long em = ((unsigned long long)__builtin_amdgcn_readfirstlane(empty_sh[1]) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane(empty_sh[0]);
    while (em) {
      const int i = __builtin_ctzll(em);
      em &= em - 1;
      epilogue(ctx(item_rank(i)));
    }
  }

  const uint16_t* kbg = a.k + (int64_t)b * a.ksb + (int64_t)g * a.ksh;
  const uint16_t* vbg = a.v + (int64_t)b * a.vsb + (int64_t)g * a.vsh;
  const uint32_t kvoff = tile_lane_offset<NW>(a.ksl), vvoff = tile_lane_offset<NW>(a.vsl);
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int e, bool is_v, int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + (uint32_t)((is_v ? 2 + buf : buf) * TILE * 2);
    const int j = __builtin_amdgcn_readfirstlane(list_sh[e]);
    const int key0 = j * KVB;
    const bool ok = j >= 0 && key0 < a.L;
    const uint16_t* base = is_v ? vbg : kbg;
    const int64_t sl = is_v ? a.vsl : a.ksl;
    if (ok && key0 + KVB <= a.L)
      issue_full_tile<KVB, NW>(base + (int64_t)key0 * sl, sl, is_v ? vvoff : kvoff, dst);
    else
      issue_tile<KVB, NW>(base + (ok ? (int64_t)key0 * sl : 0), sl, ok ? a.L - key0 : min(KVB, a.L), dst);
  };
  auto ent = [&](int e) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((int)ent_sh[e]);
  };
  // Let the Q loads land before any tile copy is issued: a use of Q inside the
  // loop would otherwise wait on every copy in flight.
  if (N == 0) return;                              // uniform over the workgroup
  if (ent(0) & 63) {                               // the first item has an empty list
    cur = ctx(__builtin_amdgcn_readfirstlane(it_r[ent(0) & 63]));
    load_q(cur);
  }
  settle(qf);
  issue(0, false, 0);
  issue(0, true, 0);
  if (N > 1) { issue(1, false, 1); issue(1, true, 1); }
  f32x16 s[KVB / 32];
  int kofs[8], vofs[8];
  k_offsets(kofs);
  v_offsets(vofs);
  auto qk = [&](int t) __attribute__((always_inline)) { qk_tile<KVB>(lds + (t & 1) * TILE, kofs, qf, s); };

  auto smpv = [&](int e, const Ctx& c, const uint16_t* Vs) __attribute__((always_inline)) {
    const int j = __builtin_amdgcn_readfirstlane(list_sh[e]);
    const int key0 = j * KVB;
    const int nk = (j < 0 || key0 >= a.L) ? 0 : min(KVB, a.L - key0);
    if (nk < KVB || (a.causal && key0 + KVB - 1 > c.wmin)) {
      int lim = nk - 1;                            // largest visible key offset of this lane's query
      if (a.causal) lim = min(lim, c.wmin + r32 - key0);
      mask_tile<KVB / 32>(s, lim);
    }
    const float msub = softmax_rescale(tile_max<KVB / 32>(s) * a.c2, m_run, l_run, o);
    softmax_pv_tile<KVB>(Vs, vofs, s, a.c2, msub, l_run, o);
  };
  // Two barriers per list entry for both groups.  Loads issued after a
  // copy (queries, output stores) only make the waits below stricter.
  auto sync_k = [&](int t) __attribute__((always_inline)) {
    if (t == 0 && N > 1) wait_loads_but<3 * IT>();
    else wait_loads_but<IT>();
    lds_barrier();
    if (t >= 1 && t + 1 < N) issue(t + 1, false, (t + 1) & 1);
  };
  auto sync_v = [&](int t) __attribute__((always_inline)) {
    if (t == 0) {
      if (N > 1) wait_loads_but<2 * IT>();
      else wait_loads_but<0>();
    } else if (t + 1 < N) {
      wait_loads_but<IT>();
    } else {
      wait_loads_but<0>();
    }
    lds_barrier();
    if (t >= 1 && t + 1 < N) issue(t + 1, true, (t + 1) & 1);
  };
  // A new item needs no zeroing of o: with the running max at -inf its first
  // visible tile rescales o by exp2(-inf) = 0 (o is always finite), and a row
  // that never sees a key is written as 0 through l = 0.
  auto restart = [&]() __attribute__((always_inline)) {
    m_run = -INFINITY;
    l_run = 0.f;
  };
  // Each role walks the entries of one item in an inner loop that loads
  // nothing the compiler can see, and handles the entry that crosses into the
  // next item in straight-line code after it: there the next queries load,
  // unconditionally (the current item's again after the last item), and are
  // awaited before the next tile copy is issued.  A load whose wait the
  // compiler cannot place on every path would make it wait for all copies in
  // flight before each K Q^T.
  int cur_it = ent(0) & 63;
  auto item_end = [&](int it) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(it_start[it + 1]);
  };
  if (grp == 0) {
    // A: K Q^T of t, then softmax + P V of t; the next item's queries load
    // during the softmax of an item's last entry
    int t = 0;
    while (true) {
      const int last = item_end(cur_it) - 1;
      for (; t < last; ++t) {
        sync_k(t);
        if (cur.busy) qk(t);
        sync_v(t);
        if (cur.busy) smpv(t, cur, lds + (2 + (t & 1)) * TILE);
      }
      sync_k(t);
      if (cur.busy) qk(t);
      sync_v(t);
      const bool more = t + 1 < N;
      const int nit_idx = more ? (ent(t + 1) & 63) : cur_it;
      const Ctx nc = ctx(__builtin_amdgcn_readfirstlane(it_r[nit_idx]));
      load_q(nc);
      if (cur.busy) smpv(t, cur, lds + (2 + (t & 1)) * TILE);
      epilogue(cur);
      restart();
      settle(qf);
      cur = nc;
      cur_it = nit_idx;
      ++t;
      if (!more) break;
    }
  } else {
    // B: softmax + P V of t - 1, then K Q^T of t; the queries of a new item
    // load once the last K Q^T of the previous one is done
    sync_k(0);
    sync_v(0);
    if (cur.busy) qk(0);
    int t = 1;
    while (true) {
      const int end = item_end(cur_it);
      for (; t < end; ++t) {                       // t - 1 and t in the same item
        sync_k(t);
        if (cur.busy) smpv(t - 1, cur, lds + (2 + ((t - 1) & 1)) * TILE);
        sync_v(t);
        if (cur.busy) qk(t);
      }
      if (t >= N) break;
      sync_k(t);                                   // t opens the next item
      const int nit_idx = ent(t) & 63;
      const Ctx nc = ctx(__builtin_amdgcn_readfirstlane(it_r[nit_idx]));
      load_q(nc);
      if (cur.busy) smpv(t - 1, cur, lds + (2 + ((t - 1) & 1)) * TILE);
      epilogue(cur);
      restart();
      settle(qf);
      cur = nc;
      cur_it = nit_idx;
      sync_v(t);
      if (cur.busy) qk(t);
      ++t;
    }
    if (cur.busy) smpv(N - 1, cur, lds + (2 + ((N - 1) & 1)) * TILE);
    epilogue(cur);
  }
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

void launch_gather(const GatherArgs& a, int kv_block, bool split, hipStream_t s) {
  if (split) {
    dim3 grid(a.items, a.NQB, a.B * a.Hkv);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<128, 4, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, 4, true>), grid, dim3(256), 0, s, a);
  } else if (a.G % 2 == 0) {
    // streaming kernel: about one workgroup per CU, each (batch, KV group) served by wpg of them
    const int BG = a.B * a.Hkv, NI = a.NQB * (a.G / 2);
    const int per_wg_max = std::min(kMaxItemsWG, kMaxListMfma / std::max(1, a.cap));
    int wpg = std::max(1, cu_count() / BG);
    wpg = std::max(wpg, (int)ceil_div(NI, per_wg_max));
    wpg = std::min(wpg, NI);
    GatherArgs b = a;
    b.wpg = wpg;
    dim3 grid(BG * wpg);
    if (kv_block == 128) hipLaunchKernelGGL((gather_stream_kernel<128>), grid, dim3(512), 0, s, b);
    else hipLaunchKernelGGL((gather_stream_kernel<64>), grid, dim3(512), 0, s, b);
  } else {
    // odd group size: one head per workgroup, 64-key tiles (two workgroups per CU)
    dim3 grid(a.B * a.Hkv * a.NQB * a.G);
    if (kv_block == 128) hipLaunchKernelGGL((gather_mfma_kernel<64, 4, false, 2>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gather_mfma_kernel<64, 4, false>), grid, dim3(256), 0, s, a);
  }
}

// The denoising step's gather with the picks inside (split mode, one query
// block): pick width U (candidates per lane = 4 U) from the number of blocks.
void launch_gather_pick(const GatherArgs& a, int kv_block, hipStream_t s) {
  dim3 grid(a.items, 1, a.B * a.Hkv);
  const int U = (int)ceil_div(a.pk.NBp, kPickThreads);
#define BSA_GP(KVB, UU) hipLaunchKernelGGL((gather_mfma_kernel<KVB, 4, true, 1, UU>), grid, dim3(256), 0, s, a)
#define BSA_GP_U(KVB)                 \
  do {                                \
    if (U <= 1) BSA_GP(KVB, 1);       \
    else if (U <= 2) BSA_GP(KVB, 2);  \
    else if (U <= 4) BSA_GP(KVB, 4);  \
    else if (U <= 8) BSA_GP(KVB, 8);  \
    else BSA_GP(KVB, 16);             \
  } while (0)
  if (kv_block == 128) BSA_GP_U(128);
  else BSA_GP_U(64);
#undef BSA_GP_U
#undef BSA_GP
}

void launch_denoise_gather(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const bsa_attn_params& p,
                           const AttnPlan& pl, const PickArgs& pk, const uint8_t* row_mask, int32_t* idx,
                           int32_t* cnt, void* ws, hipStream_t s) {
  const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
  GatherArgs a;
  a.q = static_cast<const uint16_t*>(q.data);
  a.k = static_cast<const uint16_t*>(k.data);
  a.v = static_cast<const uint16_t*>(v.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
  a.idx = idx; a.cnt = cnt; a.B = pl.B; a.cap = p.cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.G = pl.G;
  a.L = pl.L; a.Lq = pl.Lq; a.q_block = p.q_block; a.q_pos0 = p.q_pos0; a.causal = p.causal;
  a.c2 = p.scale * kLog2e;
  a.row_mask = row_mask;
  a.o = nullptr; a.o_f32 = 0; a.osb = a.osh = a.osl = 0; a.lse = nullptr;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(n * pl.D * 4));
  a.items = pl.items;
  a.wpg = 0;
  a.pk = pk;
  launch_gather_pick(a, p.kv_block, s);
}

// ------------------------------------------------------------------- host ---
bool plan_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_attn_params& p, AttnPlan& pl, int win) {
  pl.B = q.B;
  pl.Hq = q.H;
  pl.Hkv = k.H;
  pl.G = q.H / k.H;
  pl.D = q.D;
  pl.Lq = q.L;
  pl.L = k.L;
  pl.NQB = (int)ceil_div(q.L, p.q_block);
  if (p.q_block == 1) {
    pl.kind = 0;
    const int64_t toks = (int64_t)p.cap * p.kv_block;
    const bool mfma_form = q.dtype == BSA_BF16 && q.D == 128;
    pl.tok_per_item = (int)dec_slice_tokens(toks, (int64_t)pl.B * pl.Hkv * pl.NQB,
                                            mfma_form ? kDecMinSliceMfma : kDecMinSlice);
    pl.items = (int)ceil_div(toks, pl.tok_per_item) + (win > 0 ? (int)ceil_div(win, pl.tok_per_item) : 0);
    pl.qv = pl.G;
  } else if (p.q_block * pl.G <= 128 && p.q_block <= 64) {
    pl.kind = 2;
    pl.items = (int)ceil_div(p.cap, kSplitBlocks);
    pl.qv = p.q_block * pl.G;
  } else {
    pl.kind = 1;
    pl.items = 0;
    pl.qv = 0;
  }
  pl.part_bytes = 0;
  if (pl.kind != 1) {
    const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
    pl.part_bytes = align256(n * pl.D * 4) + align256(n * 2 * 4);
  }
  return true;
}

void plan_attention_counters(AttnPlan& pl) {
  pl.arrival_bytes = pl.part_bytes ? kArrivalBytes : 0;
  pl.merge_in_launch = pl.kind == 0 && pl.part_bytes && (int64_t)pl.B * pl.Hkv * pl.NQB <= kArrivalRows;
}

// Attention of each query head over its own token list (FASA technical summary
// sec. 2, focused attention: all dims, original positions): the decode split
// with one list per query head (G = 1 per list, blocks of one token), the K/V
// head found by dividing the list's head by the group size.
void plan_token_attention(const bsa_tensor& q, const bsa_tensor& k, int cap, AttnPlan& pl) {
  pl.kind = 0;
  pl.B = q.B; pl.Hq = q.H; pl.Hkv = q.H; pl.G = 1; pl.D = q.D; pl.Lq = q.L; pl.L = k.L; pl.NQB = q.L;
  pl.tok_per_item = (int)dec_slice_tokens(cap, (int64_t)pl.B * pl.Hkv * pl.NQB);
  pl.items = (int)ceil_div(cap, pl.tok_per_item);
  pl.qv = 1;
  const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
  pl.part_bytes = align256(n * pl.D * 4) + align256(n * 2 * 4);
  plan_attention_counters(pl);
}

void launch_token_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                            const int32_t* cnt, int cap, float scale, const AttnPlan& pl, const bsa_tensor& o,
                            float* lse, void* ws, hipStream_t s) {
  const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
  uint32_t* arrivals = static_cast<uint32_t*>(ws);    // the counters come first
  ws = static_cast<uint8_t*>(ws) + pl.arrival_bytes;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(n * pl.D * 4));
  DecArgs a;
  a.q = static_cast<const uint8_t*>(q.data);
  a.k = static_cast<const uint8_t*>(k.data);
  a.v = static_cast<const uint8_t*>(v.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
  a.idx = idx; a.cnt = cnt; a.cap = cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.L = pl.L;
  a.kv_block = 1; a.causal = 0; a.q_pos0 = 0; a.Lq = pl.Lq; a.items = pl.items; a.tok_per_item = pl.tok_per_item;
  a.c2 = scale * kLog2e; a.row_mask = nullptr; a.part_o = part_o; a.part_ml = part_ml;
  a.kv_div = (int)(q.H / k.H);
  if (pl.merge_in_launch) {
    a.arrivals = arrivals;
    a.o = o.data; a.o_f32 = o.dtype == BSA_F32; a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
    a.lse = lse;
  }
  launch_decode(a, q.dtype, pl.D, 1, pl.B, s);
  if (pl.merge_in_launch) return;
  CombArgs c;
  c.part_o = part_o; c.part_ml = part_ml; c.cnt = cnt; c.items = pl.items;
  c.unit_num = 1; c.unit_den = pl.tok_per_item;
  c.qvc = 256 / pl.D;
  c.Hkv = pl.Hkv; c.G = 1; c.NQB = pl.NQB; c.q_block = 1; c.Lq = pl.Lq; c.D = pl.D; c.QV = 1;
  c.row_mask = nullptr; c.o = o.data; c.osb = o.stride_b; c.osh = o.stride_h; c.osl = o.stride_l; c.lse = lse;
  launch_combine(c, o.dtype, pl.B, s);
}

void launch_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                      const int32_t* cnt, const bsa_attn_params& p, const AttnPlan& pl, const uint8_t* row_mask,
                      const bsa_tensor& o, float* lse, void* ws, hipStream_t s, int win, const float* gates) {
  const float c2 = p.scale * kLog2e;
  // the counters (if the plan has any) come first
  uint32_t* arrivals = pl.arrival_bytes ? static_cast<uint32_t*>(ws) : nullptr;
  ws = static_cast<uint8_t*>(ws) + pl.arrival_bytes;
  const bool merged = arrivals && pl.merge_in_launch;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = nullptr;
  if (pl.kind != 1) {
    const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
    part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(n * pl.D * 4));
  }
  if (pl.kind == 0) {
    DecArgs a;
    a.q = static_cast<const uint8_t*>(q.data);
    a.k = static_cast<const uint8_t*>(k.data);
    a.v = static_cast<const uint8_t*>(v.data);
    a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
    a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
    a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
    a.idx = idx; a.cnt = cnt; a.cap = p.cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.L = pl.L;
    a.kv_block = p.kv_block; a.causal = p.causal; a.q_pos0 = p.q_pos0; a.Lq = pl.Lq; a.items = pl.items;
    a.tok_per_item = pl.tok_per_item;
    a.c2 = c2; a.row_mask = row_mask; a.part_o = part_o; a.part_ml = part_ml;
    a.win = win;
    if (merged) {
      a.arrivals = arrivals;
      a.o = o.data; a.o_f32 = o.dtype == BSA_F32; a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
      a.lse = lse;
      a.gates = gates;
    }
    launch_decode(a, q.dtype, pl.D, pl.G, pl.B, s);
  } else {
    GatherArgs a;
    a.q = static_cast<const uint16_t*>(q.data);
    a.k = static_cast<const uint16_t*>(k.data);
    a.v = static_cast<const uint16_t*>(v.data);
    a.qsb = q.stride_b; a.qsh = q.stride_h; a.qsl = q.stride_l;
    a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
    a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
    a.idx = idx; a.cnt = cnt; a.B = pl.B; a.cap = p.cap; a.NQB = pl.NQB; a.Hkv = pl.Hkv; a.G = pl.G;
    a.L = pl.L; a.Lq = pl.Lq; a.q_block = p.q_block; a.q_pos0 = p.q_pos0; a.causal = p.causal; a.c2 = c2;
    a.row_mask = row_mask;
    a.o = o.data; a.o_f32 = o.dtype == BSA_F32; a.osb = o.stride_b; a.osh = o.stride_h; a.osl = o.stride_l;
    a.lse = lse; a.part_o = part_o; a.part_ml = part_ml; a.items = pl.items;
    launch_gather(a, p.kv_block, pl.kind == 2, s);
  }
  if (pl.kind != 1 && !merged) {
    CombArgs c;
    c.part_o = part_o; c.part_ml = part_ml; c.cnt = cnt; c.items = pl.items;
    if (pl.kind == 0) { c.unit_num = p.kv_block; c.unit_den = pl.tok_per_item; }
    else { c.unit_num = 1; c.unit_den = 1; c.per_item_from_count = 1; }
    c.qvc = 256 / pl.D;                          // one thread per (query vector, dim)
    c.Hkv = pl.Hkv; c.G = pl.G; c.NQB = pl.NQB; c.q_block = p.q_block; c.Lq = pl.Lq; c.D = pl.D; c.QV = pl.qv;
    c.row_mask = row_mask; c.o = o.data; c.osb = o.stride_b; c.osh = o.stride_h; c.osl = o.stride_l; c.lse = lse;
    c.win = win; c.q_pos0 = p.q_pos0; c.L = pl.L; c.gates = gates;
    launch_combine(c, o.dtype, pl.B, s);
  }
}

}  // namespace bsa
