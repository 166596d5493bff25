// Softmax-threshold decode (BLASST technical summary sec. 2: the decode kernel
// applies the same skip rule as prefill, and since decode is bound by memory
// the saving is the V load of a skipped block).
//
// Each head walks the tiles of 64 keys from the newest down with a running
// max m, keeping a tile when it is the first or its max tm trails m by less
// than ln(1 / lambda).  A skipped tile has tm < m, so it could not have raised
// m: the running max before tile j is the max of all newer tiles' maxima,
// kept or not.  The sequential walk therefore splits into independent work:
//   1. scores_kernel: one workgroup per (slice of kv_split keys, KV group);
//      K of the slice streams through the matrix cores, and q.k for the G
//      heads of the group (log2 units), each tile's max and the slice's max
//      go to the workspace;
//   2. pv_kernel: one workgroup per (chunk of up to 4 tiles, KV group); the
//      max over all newer tiles decides every (head, tile) of the chunk; V is
//      loaded only for tiles some head keeps (the G heads share each load,
//      NSA implementation-challenges section), and each head sums
//      2^(s - m_c) v over its kept keys, m_c being its largest kept tile max
//      in the chunk.  The walk keeps most tiles near the newest end, so small
//      chunks spread that work over many compute units;
//   3. combine_kernel: per head, the chunks' maxima in one round trip, then
//      the partial sums of the chunks that kept anything, merged in order.
//
// The end of the file holds the token selection on a subset of frequency
// chunks (FASA), which reuses the scores kernel with a chunk mask.
#include "common.h"
#include "internal.h"
#include "split.h"

namespace bsa {

constexpr int kTDecTile = 64;           // keys per tile
constexpr int kTDecMaxSplit = 2048;     // keys per slice, at most
constexpr int kTDecChunkTiles = 4;     // tiles per decision / P V chunk, at most
constexpr int kTDecMaxChunks = 4096;    // chunks per head the combine takes

struct TDecArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t qsb, qsh, ksb, ksh, ksl, vsb, vsh, vsl;
  int Hkv, G, L, Lpad, split, nsplit, ntiles, ctiles, nchunk;   // ctiles: tiles per chunk
  float c2;                             // scale * log2(e)
  float ln_lam2;                        // ln(lambda) * log2(e); -inf for lambda = 0
  float* scores;                        // [B][Hkv][G][Lpad], log2 units; Lpad = L rounded up to 4
  float* tmax;                          // [B][Hkv][G][ntiles]
  float* smax;                          // [B][Hkv][G][nsplit] max over a slice's tiles
  float* part_o;                        // [B][Hkv][nchunk][G][D] (written only where the chunk kept a tile)
  float* part_ml;                       // [B][Hkv][nchunk][G][2] (m: largest kept tile max or -inf; l)
  int32_t* part_cnt;                    // [B][Hkv][nchunk][G] kept tiles
  int32_t* kept;                        // [B][Hq] kept tiles per head, or null
  uint8_t* keep_map;                    // [B][Hq][ntiles] or null
  const uint8_t* fc_mask;               // token scoring: [Hq][64] frequency chunks in use (D = 128), or null
  int layout;                           // RoPE layout naming the two dims of each chunk
  void* o;                              // [B][Hq][1][D], bf16 or f32
  int64_t osb, osh;
  float* lse;                           // [B][Hq][1]
};

// Scores of one slice: q.k (log2 units) for the G heads of the group, and the
// max of each tile, into the workspace.  The products run on the matrix
// cores: S = K Q^T with v_mfma_f32_16x16x32_bf16, 16 keys by 16 columns (the
// G heads, the rest zero) per product, 4 products over the 128 dims.  Each
// lane's A operand is 8 consecutive dims of one key row, i.e. one 16-byte
// load straight from global memory; a wave walks its chunks of 16 keys two
// batches deep, so one batch of loads is in flight while the other is used.
template <int G>
__global__ __launch_bounds__(512) void tdec_scores_kernel(TDecArgs a) {
  constexpr int T = kTDecTile, CH = 16, NB = 2;     // keys per chunk, chunks per batch
  constexpr int NW = 8;                             // waves
  __shared__ float sc[G][kTDecMaxSplit];
  __shared__ float tmx[G][kTDecMaxSplit / kTDecTile];

  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;        // operand column / k-group of this lane
  const int s0 = split * a.split;
  const int n = min(a.split, a.L - s0);             // keys of this slice (>= 1)
  const int nt = (n + T - 1) / T;

  // Q^T operand: column = head (zero past G), k = dims 32 ks + 8 kq + 0..7
  // (all loads of q and of the chunk mask are requested before any is used: loads under a
  // branch, or used as they arrive, would each wait for the one before)
  bf16x8 qb[4];
  u32x4 qw[4];
  const int hq = g * G + min(col, G - 1);           // columns past G load a valid row, then zeroed
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qw[ks] = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.qsb + (int64_t)hq * a.qsh + 32 * ks + 8 * kq) * 2);
  if (a.fc_mask) {                                  // uniform
    // token scoring on a subset of frequency chunks: zero the query dims of the other chunks
    const uint8_t* fm = a.fc_mask + (int64_t)hq * 64;
    uint8_t mb[4][4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * ks + 8 * kq + 2 * e;             // dims d, d + 1 of word e
        mb[ks][e][0] = fm[a.layout == BSA_ROPE_HALF ? (d & 63) : (d >> 1)];
        mb[ks][e][1] = fm[a.layout == BSA_ROPE_HALF ? ((d + 1) & 63) : (d >> 1)];
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[ks][e] &= (mb[ks][e][0] ? 0x0000FFFFu : 0u) | (mb[ks][e][1] ? 0xFFFF0000u : 0u);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (col >= G) qw[ks] = u32x4{0u, 0u, 0u, 0u};
    qb[ks] = __builtin_bit_cast(bf16x8, qw[ks]);
  }
  const uint8_t* kb = a.k + ((int64_t)b * a.ksb + (int64_t)g * a.ksh + (int64_t)s0 * a.ksl) * 2;
  const int nch = (nt * T) / CH;                    // chunks of the slice's tiles
  const int per_wave = (nch + NW - 1) / NW;         // chunks w, w + NW, ...
  const int nbatch = (per_wave + NB - 1) / NB;
  // loads are unconditional (chunks past the slice re-read its last chunk) so
  // that a batch issues as one group; the products skip those chunks
  auto load_batch = [&](int j, bf16x8 (&dst)[NB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = min(w + NW * (j * NB + u), nch - 1);
      const int key = min(c * CH + col, n - 1);     // rows past the slice repeat its last key
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        dst[u][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(kb + ((int64_t)key * a.ksl + 32 * ks + 8 * kq) * 2));
    }
  };
  auto use_batch = [&](int j, const bf16x8 (&src)[NB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = w + NW * (j * NB + u);
      if (c >= nch) continue;                       // uniform over the wave
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(src[u][ks], qb[ks], acc, 0, 0, 0);
      // lane holds keys c*16 + 4 kq + r (r = 0..3) of head col
      if (col < G) {
        const int k0 = c * CH + 4 * kq;
        f32x4 out;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = k0 + r < n ? acc[r] * a.c2 : -INFINITY;
        *reinterpret_cast<f32x4*>(&sc[col][k0]) = out;
      }
    }
  };
  bf16x8 ka[NB][4], kbuf[NB][4];
  if (nbatch > 0) load_batch(0, ka);
  for (int j = 0; j < nbatch; j += 2) {
    if (j + 1 < nbatch) load_batch(j + 1, kbuf);
    use_batch(j, ka);
    if (j + 2 < nbatch) load_batch(j + 2, ka);
    if (j + 1 < nbatch) use_batch(j + 1, kbuf);
  }
  __syncthreads();
  // scores out (keys of the slice, 16-byte stores), the tile maxima, and the
  // slice's max per head (what the later slices' walks start from)
  const int64_t hb = ((int64_t)b * a.Hkv + g) * G;
  for (int i = tid; i < G * (n / 4); i += NW * 64) {
    const int h = i / (n / 4), c = i - h * (n / 4);
    *reinterpret_cast<f32x4*>(a.scores + (hb + h) * a.Lpad + s0 + 4 * c) =
        *reinterpret_cast<const f32x4*>(&sc[h][4 * c]);
  }
  for (int i = tid; i < G * (n % 4); i += NW * 64) {
    const int h = i / (n % 4), c = n - n % 4 + i % (n % 4);
    a.scores[(hb + h) * a.Lpad + s0 + c] = sc[h][c];
  }
  for (int vi = tid / 4; vi < G * nt; vi += NW * 16) {
    const int h = vi / nt, t = vi - h * nt, qq = tid & 3;
    const float* r = &sc[h][t * T + qq * (T / 4)];
    float mx = r[0];
#pragma unroll
    for (int i = 1; i < T / 4; ++i) mx = fmaxf(mx, r[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    if (qq == 0) {
      a.tmax[(hb + h) * a.ntiles + s0 / T + t] = mx;
      tmx[h][t] = mx;
    }
  }
  __syncthreads();
  if (tid < G) {
    float mx = -INFINITY;
    for (int t = 0; t < nt; ++t) mx = fmaxf(mx, tmx[tid][t]);
    a.smax[(hb + tid) * a.nsplit + split] = mx;
  }
}

// Decisions, V and P V of one chunk (up to 4 tiles), four waves.  Round trip
// one brings the chunk's scores (into LDS, key-major), the maxima of its
// slice's tiles from the chunk on, and the maxima of all newer slices; the
// decisions follow -- tile j of head h is kept iff its max tm passes the test
// against the max of every newer tile -- and then the V loads of all kept
// tiles at once.  The waves split the head dims (32 each: 8 lanes x 4 dims
// per key row, 8 keys per pass), so each wave walks every kept tile.  While
// the loads are in flight the workgroup turns the kept scores into
// p = 2^(s - m_c) in place (0 for a tile or key the head does not keep).
// CHECK = false (lambda = 0) compiles the skip test out: every finite tile is
// kept and the newer tiles' maxima are not read.
template <int G, bool CHECK>
__global__ __launch_bounds__(256) void tdec_pv_kernel(TDecArgs a) {
  constexpr int D = 128, T = kTDecTile, NW = 4, NT = 256;
  constexpr int MAXT = kTDecMaxSplit / T;           // tiles per slice, at most 32
  constexpr int MAXC = kTDecChunkTiles;
  constexpr int NPAIR = (2 * G + 3) / 4;            // ballots of (head, tile) pairs: 2 heads x 32 tiles each
  constexpr int DW = D / NW, LPK = DW / 4;          // dims per wave, lanes per key row
  constexpr int KPP = 64 / LPK, PPT = T / KPP;      // keys per pass, passes per tile
  __shared__ __align__(16) float sc[MAXC * T * G];  // [key][head]: scores, then p
  __shared__ float tmx[G][MAXT];
  __shared__ float newer_sh[G];

  const int chunk = a.nchunk - 1 - (int)blockIdx.x;         // newest chunks (most kept tiles) first
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int t0 = chunk * a.ctiles;                          // first tile of the chunk
  const int s0 = t0 * T;
  const int n = min(a.ctiles * T, a.L - s0);                // keys of the chunk
  const int nt = (n + T - 1) / T;
  const int sp = s0 / a.split;                              // the slice holding the chunk
  const int ntail = min((sp + 1) * (a.split / T), a.ntiles) - t0;   // tiles from t0 to the slice's end
  const int nq = (n + 3) / 4;                               // 16-byte score chunks per head row
  const int64_t hb = ((int64_t)b * a.Hkv + g) * G;

  // ---- round trip 1
  {
    constexpr int NR = (MAXC * T / 4 * G + NT - 1) / NT;
    f32x4 sv[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int i = min(tid + NT * r, G * nq - 1);
      const int h = i / nq, c = i - h * nq;
      sv[r] = *reinterpret_cast<const f32x4*>(a.scores + (hb + h) * a.Lpad + s0 + 4 * c);
    }
    float tv = -INFINITY;
    if (tid < G * MAXT) {
      const int h = tid / MAXT, j = tid - h * MAXT;
      if (j < ntail) tv = a.tmax[(hb + h) * a.ntiles + t0 + j];
    }
    float nv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      nv[h] = -INFINITY;
      if (CHECK && w == NW - 1)
        for (int q = sp + 1 + lane; q < a.nsplit; q += 64) nv[h] = fmaxf(nv[h], a.smax[(hb + h) * a.nsplit + q]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int i = tid + NT * r;
      if (i < G * nq) {
        const int h = i / nq, c = i - h * nq;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[(4 * c + e) * G + h] = sv[r][e];
      }
    }
    if (tid < G * MAXT) tmx[tid / MAXT][tid % MAXT] = tv;
    if (CHECK && w == NW - 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m = wave_max_dpp(nv[h]);
        if (lane == 0) newer_sh[h] = m;
      }
    }
  }
  __syncthreads();

  // ---- decisions: ballot r covers heads 2r (lanes 0-31) and 2r + 1 (lanes 32-63), lane % 32 = tile - t0
  uint32_t kb[G];
  float mk[G];
  uint32_t any = 0u;
#pragma unroll
  for (int r = 0; r < NPAIR; ++r) {
    const int h = 2 * r + lane / 32, j = lane % 32;
    const bool valid = h < G && j < ntail;
    const float tm = valid ? tmx[h < G ? h : 0][j] : -INFINITY;
    const bool mine = valid && j < nt;                      // a tile of this chunk
    bool keep = mine && tm > -INFINITY;
    if constexpr (CHECK) {
      // max over the slice's tiles after j (shuffles stay inside each 32-lane half)
      float incl = tm;
#pragma unroll
      for (int sft = 1; sft < 32; sft <<= 1) incl = fmaxf(incl, __shfl_down(incl, sft, 32));
      float excl = __shfl_down(incl, 1, 32);
      if (j == 31) excl = -INFINITY;
      const float M = fmaxf(valid ? newer_sh[h] : -INFINITY, excl);
      keep = keep && (M == -INFINITY || tm - M >= a.ln_lam2);
    }
    const uint64_t bal = __ballot(keep);
    float x = keep ? tm : -INFINITY;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 32));
    const float x0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 0));
    const float x1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 32));
    if (2 * r < G) { kb[2 * r] = (uint32_t)bal; mk[2 * r] = x0; any |= (uint32_t)bal; }
    if (2 * r + 1 < G) { kb[2 * r + 1] = (uint32_t)(bal >> 32); mk[2 * r + 1] = x1; any |= (uint32_t)(bal >> 32); }
    if (w == 0 && mine && a.keep_map) a.keep_map[(hb + h) * a.ntiles + t0 + j] = keep ? 1 : 0;
  }
  float msub[G];
#pragma unroll
  for (int h = 0; h < G; ++h) msub[h] = mk[h] == -INFINITY ? 0.f : mk[h];

  // ---- V of the kept tiles, p in place, P V
  const int kw = lane / LPK, dl = w * DW + (lane % LPK) * 4;   // key row of the pass, first dim
  // uniform base of the chunk's V rows, 32-bit lane offsets (the host bounds the row stride)
  const uint8_t* vb = a.v + ((int64_t)b * a.vsb + (int64_t)g * a.vsh + (int64_t)s0 * a.vsl) * 2;
  const uint32_t rowb = (uint32_t)a.vsl * 2u;
  float acc[G][4], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
  }
  if (any) {                                         // the same on every wave
    u32x2 vv[MAXC][PPT];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (!((any >> c) & 1u)) continue;
#pragma unroll
      for (int p = 0; p < PPT; ++p) {
        const uint32_t kr = (uint32_t)min(c * T + KPP * p + kw, n - 1);
        vv[c][p] = *reinterpret_cast<const u32x2*>(vb + (kr * rowb + (uint32_t)dl * 2u));
      }
    }
    // p for every (key, head) of every kept tile, keys past the chunk included (p = 0)
#pragma unroll
    for (int r = 0; r < MAXC * T * G / NT; ++r) {
      const int e = tid + NT * r;
      const int c = e / (T * G), ke = e - c * (T * G);
      const int h = ke % G, key = c * T + ke / G;
      if ((any >> c) & 1u) {
        uint32_t kbh = 0u;
        float ms = 0.f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          if (hh == h) { kbh = kb[hh]; ms = msub[hh]; }
        float* ps = &sc[key * G + h];
        const bool use = ((kbh >> c) & 1u) && key < n;
        *ps = use ? fast_exp2(*ps - ms) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (!((any >> c) & 1u)) continue;
#pragma unroll
      for (int p = 0; p < PPT; ++p) {
        const int key = c * T + KPP * p + kw;
        float pr[G];
        if constexpr (G >= 4) {
#pragma unroll
          for (int q4 = 0; q4 < G / 4; ++q4) {
            const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sc[key * G + 4 * q4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pr[4 * q4 + e] = x4[e];
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pr[h] = sc[key * G + h];
        }
        const float vx[4] = {__uint_as_float(vv[c][p][0] << 16), __uint_as_float(vv[c][p][0] & 0xFFFF0000u),
                             __uint_as_float(vv[c][p][1] << 16), __uint_as_float(vv[c][p][1] & 0xFFFF0000u)};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (w == 0 && lane % LPK == 0) lsum[h] += pr[h];   // each key once
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[h][e] = fmaf(pr[h], vx[e], acc[h][e]);
        }
      }
    }
  }

  // ---- sums over the 8 key rows of the wave; each wave owns its dims
  const int64_t pbase = (((int64_t)b * a.Hkv + g) * a.nchunk + chunk) * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (mk[h] == -INFINITY) continue;                // uniform: the combine reads no o for this chunk
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = acc[h][e];
      x += dpp_f32<0x128>(0.f, x);                  // row_ror:8: lanes i and i ^ 8
      acc[h][e] = groups_sum<16>(x);
    }
    if (lane < LPK)
      *reinterpret_cast<f32x4*>(a.part_o + (pbase + h) * D + dl) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
  }
  if (w == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l = wave_sum_dpp(lsum[h]);
      if (lane == 0) {
        a.part_ml[(pbase + h) * 2] = mk[h];
        a.part_ml[(pbase + h) * 2 + 1] = l;
        a.part_cnt[pbase + h] = __popc(kb[h]);
      }
    }
  }
}

// Merge of one head's chunks in ascending order.  Round trip one brings every
// chunk's (m, l) and kept count; the chunks that kept a tile are compacted
// (ballots, one scan of the per-wave counts); round trip two brings their
// partial O (four threads per dim share the list); the global max M is known
// first, so every term is scaled once by 2^(m - M).
template <int ODT>
__global__ __launch_bounds__(512) void tdec_combine_kernel(TDecArgs a) {
  constexpr int D = 128, NT = 512, NW = 8, MAXC = kTDecMaxChunks, NI = MAXC / NT;
  constexpr int PARTS = NT / D, BJ = 32;             // threads per dim, chunks per batch per thread
  __shared__ float ms[MAXC], ls[MAXC];
  __shared__ int list[MAXC];
  __shared__ int goff[MAXC / 64];
  __shared__ float redm[NW];
  __shared__ int redk[NW], nlist;
  __shared__ float part_acc[PARTS - 1][D], part_l[PARTS - 1];

  const int G = a.G, Hq = a.Hkv * G;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh - b * Hq, g = h / G, hl = h - g * G;
  const int64_t base = ((int64_t)b * a.Hkv + g) * a.nchunk;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nc = a.nchunk, ni = (nc + NT - 1) / NT;

  // ---- round trip 1: (m, l) and counts of every chunk
  f32x2 mlv[NI];
  int cv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i < ni) {
      const int64_t pi = (base + min(tid + NT * i, nc - 1)) * G + hl;
      mlv[i] = *reinterpret_cast<const f32x2*>(a.part_ml + pi * 2);
      cv[i] = a.part_cnt[pi];
    }
  }
  float mx = -INFINITY;
  int kt = 0;
  uint64_t bal[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    bal[i] = 0;
    if (i < ni) {
      const int c = tid + NT * i;
      const bool valid = c < nc;
      const float m = valid ? mlv[i][0] : -INFINITY;
      if (valid) { ms[c] = m; ls[c] = mlv[i][1]; kt += cv[i]; }
      mx = fmaxf(mx, m);
      bal[i] = __ballot(m > -INFINITY);
      if (lane == 0) goff[i * NW + w] = __popcll(bal[i]);      // chunks 64 (NW i + w) ...
    }
  }
  mx = wave_max_dpp(mx);
  const int ktw = (int)wave_sum_dpp((float)kt);              // counts stay far below 2^24
  if (lane == 0) { redm[w] = mx; redk[w] = ktw; }
  __syncthreads();
  if (w == 0) {                                              // exclusive scan of the group counts
    const int ng = ni * NW;
    const uint32_t x = lane < ng ? (uint32_t)goff[lane] : 0u;
    const uint32_t incl = wave_incl_scan_dpp(x);
    if (lane < ng) goff[lane] = (int)(incl - x);
    if (lane == 63) nlist = (int)incl;
  }
  float M = redm[0];
  int ktot = redk[0];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) { M = fmaxf(M, redm[ww]); ktot += redk[ww]; }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i < ni && ((bal[i] >> lane) & 1ull)) {
      const int below = __popcll(bal[i] & ((1ull << lane) - 1ull));
      list[goff[i * NW + w] + below] = tid + NT * i;
    }
  }
  __syncthreads();

  // ---- round trip 2: partial O of the listed chunks
  const int K = nlist;
  const int d = tid % D, part = tid / D;
  float acc = 0.f, lsum = 0.f;
  for (int j0 = 0; j0 * PARTS < K; j0 += BJ) {
    float ov[BJ];
    int cl[BJ];
#pragma unroll
    for (int u = 0; u < BJ; ++u) {
      const int e = min((j0 + u) * PARTS + part, K - 1);
      cl[u] = list[e];
      ov[u] = a.part_o[((base + cl[u]) * G + hl) * D + d];
    }
#pragma unroll
    for (int u = 0; u < BJ; ++u) {
      if ((j0 + u) * PARTS + part < K) {
        const float wgt = fast_exp2(ms[cl[u]] - M);
        acc = fmaf(ov[u], wgt, acc);
        lsum = fmaf(ls[cl[u]], wgt, lsum);
      }
    }
  }
  if (part > 0) {
    part_acc[part - 1][d] = acc;
    if (d == 0) part_l[part - 1] = lsum;
  }
  __syncthreads();
  if (part == 0) {
#pragma unroll
    for (int q = 0; q < PARTS - 1; ++q) { acc += part_acc[q][d]; lsum += part_l[q]; }
    const float out = lsum > 0.f ? acc / lsum : 0.f;
    const int64_t oi = (int64_t)b * a.osb + (int64_t)h * a.osh + d;
    if (ODT == BSA_BF16) reinterpret_cast<uint16_t*>(a.o)[oi] = (uint16_t)f32_to_bf16(out);
    else reinterpret_cast<float*>(a.o)[oi] = out;
    if (d == 0) {
      a.lse[(int64_t)b * Hq + h] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
      if (a.kept) a.kept[(int64_t)b * Hq + h] = ktot;
    }
  }
}

// tiles per decision chunk: 4 when a slice holds whole chunks of 4, else 2 or 1
static int tdec_chunk_tiles(int kv_split) {
  const int t = kv_split / kTDecTile;
  return t % 4 == 0 ? 4 : (t % 2 == 0 ? 2 : 1);
}

static size_t tdec_sizes(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t (&sz)[6]) {
  const int64_t nsplit = ceil_div(k.L, kv_split), ntiles = ceil_div(k.L, kTDecTile);
  const int64_t nchunk = ceil_div(ntiles, tdec_chunk_tiles(kv_split));
  const size_t heads = (size_t)q.B * q.H;            // B * Hkv * G
  const size_t n = heads * nchunk;
  sz[0] = align256(heads * ((k.L + 3) & ~3LL) * 4);    // scores, rows padded to 16 bytes
  sz[1] = align256(heads * ntiles * 4);                // tile maxima
  sz[2] = align256(n * q.D * 4);                       // partial O
  sz[3] = align256(n * 2 * 4);                         // partial (m, l)
  sz[4] = align256(n * 4);                             // kept tiles per chunk
  sz[5] = align256(heads * nsplit * 4);                // slice maxima
  return sz[0] + sz[1] + sz[2] + sz[3] + sz[4] + sz[5];
}

bool plan_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t& bytes) {
  size_t sz[6];
  bytes = tdec_sizes(q, k, kv_split, sz);
  return ceil_div(ceil_div(k.L, kTDecTile), tdec_chunk_tiles(kv_split)) <= kTDecMaxChunks;
}

void launch_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, float scale,
                             float lambda, int kv_split, const bsa_tensor& o, float* lse, int32_t* kept,
                             uint8_t* keep_map, void* ws, hipStream_t s) {
  const int G = (int)(q.H / k.H);
  TDecArgs a;
  a.q = static_cast<const uint8_t*>(q.data);
  a.k = static_cast<const uint8_t*>(k.data);
  a.v = static_cast<const uint8_t*>(v.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.vsb = v.stride_b; a.vsh = v.stride_h; a.vsl = v.stride_l;
  a.Hkv = (int)k.H; a.G = G; a.L = (int)k.L; a.Lpad = (int)((k.L + 3) & ~3LL); a.split = kv_split;
  a.nsplit = (int)ceil_div(k.L, kv_split);
  a.ntiles = (int)ceil_div(k.L, kTDecTile);
  a.ctiles = tdec_chunk_tiles(kv_split);
  a.nchunk = (int)ceil_div(a.ntiles, a.ctiles);
  a.c2 = scale * kLog2e;
  a.ln_lam2 = lambda > 0.f ? logf(lambda) * kLog2e : -INFINITY;
  size_t sz[6];
  tdec_sizes(q, k, kv_split, sz);
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.scores = reinterpret_cast<float*>(p);
  p += sz[0];
  a.tmax = reinterpret_cast<float*>(p);
  p += sz[1];
  a.part_o = reinterpret_cast<float*>(p);
  p += sz[2];
  a.part_ml = reinterpret_cast<float*>(p);
  p += sz[3];
  a.part_cnt = reinterpret_cast<int32_t*>(p);
  p += sz[4];
  a.smax = reinterpret_cast<float*>(p);
  a.kept = kept;
  a.keep_map = keep_map;
  a.fc_mask = nullptr;
  a.layout = 0;
  a.o = o.data; a.osb = o.stride_b; a.osh = o.stride_h;
  a.lse = lse;
  const dim3 gs(a.nsplit, q.B * k.H), gp(a.nchunk, q.B * k.H);
#define BSA_TDEC(GG)                                                                  \
  hipLaunchKernelGGL(tdec_scores_kernel<GG>, gs, dim3(512), 0, s, a);                 \
  if (lambda > 0.f) hipLaunchKernelGGL((tdec_pv_kernel<GG, true>), gp, dim3(256), 0, s, a); \
  else hipLaunchKernelGGL((tdec_pv_kernel<GG, false>), gp, dim3(256), 0, s, a)
  switch (G) {
    case 1: BSA_TDEC(1); break;
    case 2: BSA_TDEC(2); break;
    case 4: BSA_TDEC(4); break;
    default: BSA_TDEC(8); break;
  }
#undef BSA_TDEC
  if (o.dtype == BSA_BF16) hipLaunchKernelGGL(tdec_combine_kernel<BSA_BF16>, dim3(q.B * q.H), dim3(512), 0, s, a);
  else hipLaunchKernelGGL(tdec_combine_kernel<BSA_F32>, dim3(q.B * q.H), dim3(512), 0, s, a);
}

// ----------------------------------------------------------------------------
// Token importance on a subset of frequency chunks (FASA technical summary
// sec. 2, token importance prediction: q.k over the dims of a head's dominant
// chunks only) and the top-N tokens of each head.
//
// Scores come from the scores kernel above with the other chunks' query dims
// zeroed.  The top N of a head's L scores (ties to the lower token) take two
// passes of one selection kernel, so that many CUs share a head:
//   1. each of P parts of kTokPart tokens keeps its own top N (a global top-N
//      token is in its part's top N under the same tie rule);
//   2. one workgroup per head selects the top N of the P x N candidates.
// A workgroup holds its elements in registers as order-preserving keys
// (larger score, larger key; 0 marks no token), finds the N-th largest key
// two bits at a time with 16 counting steps, and places the chosen elements in their
// original order (ascending tokens) with two block scans.
constexpr int kTokPart = 4096;          // tokens per first-pass part
constexpr int kTokMaxBudget = 2048;     // tokens per head, at most
constexpr int kTokMaxCand = 16384;      // first-pass candidates per head, at most
constexpr int kTokBits = 2;             // bits of the N-th key found per counting step (divides 32)
constexpr int kTokKeysPerGroup = 8;     // keys whose ballots are taken before they are summed

struct TopkArgs {
  const float* scores;                  // pass 1: [rows][Lpad]
  const uint32_t* in_keys;              // pass 2: [rows][P * N] candidates (0: none)
  const int32_t* in_toks;
  uint32_t* out_keys;                   // pass 1 output: [rows][P][N]
  int32_t* out_toks;
  int32_t* idx;                         // pass 2 output: [rows][N] and counts [rows]
  int32_t* cnt;
  int Lpad, L, N, P;
};

template <int NT, int PER, bool FIRST>
__global__ __launch_bounds__(NT) void token_topk_kernel(TopkArgs a) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t wsum[2][NW];                   // double-buffered: one barrier per block sum
  __shared__ uint32_t wsum3[2][(1 << kTokBits) - 1][NW];   // the same for the counts of one step
  const int part = blockIdx.x, row = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int e0 = tid * PER;                          // this thread's first element
  uint32_t key[PER];
  int32_t tk[FIRST ? 1 : PER];
  int n_elem, Ne;
  if (FIRST) {
    const int t0 = part * kTokPart;                  // first token of the part
    n_elem = min(kTokPart, a.L - t0);
    Ne = min(a.N, n_elem);
    const float* sr = a.scores + (int64_t)row * a.Lpad + t0;
    const int lim = n_elem - e0;                     // element e is in the part iff e < lim
    const int cl = a.Lpad - t0 - 4;                  // last 16-byte chunk of the row from the part's start
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sr + min(e0 + 4 * c, cl));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = __float_as_uint(x[e]);
        key[4 * c + e] = 4 * c + e < lim ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
      }
    }
  } else {
    n_elem = a.P * a.N;
    Ne = min(a.N, a.L);
    const uint32_t* kr = a.in_keys + (int64_t)row * n_elem;
    const int32_t* tr = a.in_toks + (int64_t)row * n_elem;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = min(e0 + e, n_elem - 1);
      const uint32_t kk = kr[i];
      key[e] = e0 + e < n_elem ? kk : 0u;
      tk[e] = tr[i];
    }
  }
  // Block-wide sum (exact: counts stay far below 2^24) and exclusive scan of one
  // value per thread.  Call k uses wsum[k & 1]: a wave can only write a buffer
  // again two calls later, after every wave has passed the barrier between.
  int call = 0;
  auto block_sum = [&](uint32_t v) __attribute__((always_inline)) {
    const float ws = wave_sum_dpp((float)v);
    uint32_t* buf = wsum[call++ & 1];
    if (lane == 0) buf[w] = (uint32_t)ws;
    __syncthreads();
    uint32_t tot = 0u;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) tot += buf[ww];
    return tot;
  };
  auto block_excl = [&](uint32_t v) __attribute__((always_inline)) {
    const uint32_t inc = wave_incl_scan_dpp(v);
    uint32_t* buf = wsum[call++ & 1];
    if (lane == 63) buf[w] = inc;
    __syncthreads();
    uint32_t before = 0u;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      if (ww < w) before += buf[ww];
    return before + inc - v;
  };
  // The N-th largest key: the largest x with at least N keys >= x, two bits a
  // step (the counts at the three candidates x | 1, 2, 3 << shift, reduced
  // together: their latencies overlap).
  uint32_t tau = 0u;
  int call3 = 0;
  constexpr int NC = (1 << kTokBits) - 1;            // candidates per step
#pragma unroll 1
  for (int shift = 32 - kTokBits; shift >= 0; shift -= kTokBits) {
    // the wave's counts straight from ballots: one compare per (key, candidate), the
    // population counts and sums on the scalar unit, no cross-lane reduction
    uint32_t ws[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) ws[j] = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
#pragma unroll
      for (int j = 0; j < NC; ++j)
        ws[j] += (uint32_t)__popcll(__ballot(key[e] >= (tau | ((uint32_t)(j + 1) << shift))));
      // a few keys at a time: the compiler would otherwise hold every ballot in scalar registers
      if (e % kTokKeysPerGroup == kTokKeysPerGroup - 1) __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t (*buf)[NW] = wsum3[call3++ & 1];
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < NC; ++j) buf[j][w] = ws[j];
    }
    __syncthreads();
    // counts fall with the candidate: take the largest one that still has N keys
    uint32_t dg = 0u;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      uint32_t t = 0u;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) t += buf[j][ww];
      dg = t >= (uint32_t)Ne ? (uint32_t)(j + 1) : dg;
    }
    tau |= dg << shift;
  }
  uint32_t n_gt = 0u, n_eq = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    n_gt += key[e] > tau;
    n_eq += key[e] == tau;
  }
  const uint32_t need = (uint32_t)Ne - block_sum(n_gt);   // ties at the N-th key still to take
  const uint32_t eq_before = block_excl(n_eq);
  const uint32_t take = need > eq_before ? min(need - eq_before, n_eq) : 0u;
  uint32_t pos = block_excl(n_gt + take);
  uint32_t taken = 0u;
  if (FIRST) {
    const int64_t ob = ((int64_t)row * a.P + part) * a.N;
    int tok = part * kTokPart + e0;
    asm volatile("" : "+v"(tok));                    // one running token index, not PER precomputed ones
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool eq = key[e] == tau && taken < take;
      if (key[e] > tau || eq) {
        a.out_keys[ob + pos] = key[e];
        a.out_toks[ob + pos] = tok;
        ++pos;
      }
      taken += eq;
      ++tok;
    }
    for (int i = Ne + tid; i < a.N; i += NT) a.out_keys[ob + i] = 0u;   // unused slots: no token
  } else {
    int32_t* out = a.idx + (int64_t)row * a.N;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool eq = key[e] == tau && taken < take;
      if (key[e] > tau || eq) out[pos++] = tk[e];
      taken += eq;
    }
    if (tid == 0) a.cnt[row] = Ne;
  }
}

static void tok_plan(const bsa_tensor& k, int budget, int& P) { P = (int)ceil_div(k.L, kTokPart); (void)budget; }

static size_t tok_sizes(const bsa_tensor& q, const bsa_tensor& k, int budget, size_t (&sz)[5]) {
  const size_t heads = (size_t)q.B * q.H;
  int P;
  tok_plan(k, budget, P);
  sz[0] = align256(heads * ((k.L + 3) & ~3LL) * 4);                 // scores
  sz[1] = align256(heads * ceil_div(k.L, kTDecTile) * 4);           // tile maxima (written, unused)
  sz[2] = align256(heads * ceil_div(k.L, kTDecMaxSplit) * 4);       // slice maxima (written, unused)
  sz[3] = align256(heads * (size_t)P * budget * 4);                 // first-pass keys
  sz[4] = align256(heads * (size_t)P * budget * 4);                 // first-pass tokens
  return sz[0] + sz[1] + sz[2] + sz[3] + sz[4];
}

bool token_select_supported(const bsa_tensor& k, int budget) {
  int P;
  tok_plan(k, budget, P);
  return budget <= kTokMaxBudget && (int64_t)P * budget <= kTokMaxCand;
}

size_t token_select_workspace(const bsa_tensor& q, const bsa_tensor& k, int budget) {
  size_t sz[5];
  return tok_sizes(q, k, budget, sz);
}

void launch_token_select(const bsa_tensor& q, const bsa_tensor& k, const uint8_t* fc_mask, int layout, int budget,
                         int32_t* idx, int32_t* cnt, float* scores_out, void* ws, hipStream_t s) {
  const int G = (int)(q.H / k.H);
  TDecArgs a{};
  a.q = static_cast<const uint8_t*>(q.data);
  a.k = static_cast<const uint8_t*>(k.data);
  a.qsb = q.stride_b; a.qsh = q.stride_h;
  a.ksb = k.stride_b; a.ksh = k.stride_h; a.ksl = k.stride_l;
  a.Hkv = (int)k.H; a.G = G; a.L = (int)k.L; a.Lpad = (int)((k.L + 3) & ~3LL); a.split = kTDecMaxSplit;
  a.nsplit = (int)ceil_div(k.L, kTDecMaxSplit);
  a.ntiles = (int)ceil_div(k.L, kTDecTile);
  a.c2 = 1.f;                                        // plain q.k
  size_t sz[5];
  tok_sizes(q, k, budget, sz);
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.scores = scores_out ? scores_out : reinterpret_cast<float*>(p);
  a.tmax = reinterpret_cast<float*>(p + sz[0]);
  a.smax = reinterpret_cast<float*>(p + sz[0] + sz[1]);
  a.fc_mask = fc_mask;
  a.layout = layout;
  const dim3 gs(a.nsplit, q.B * k.H);
  switch (G) {
    case 1: hipLaunchKernelGGL(tdec_scores_kernel<1>, gs, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL(tdec_scores_kernel<2>, gs, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(tdec_scores_kernel<4>, gs, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL(tdec_scores_kernel<8>, gs, dim3(512), 0, s, a); break;
  }
  TopkArgs t{};
  t.scores = a.scores;
  t.in_keys = reinterpret_cast<const uint32_t*>(p + sz[0] + sz[1] + sz[2]);
  t.in_toks = reinterpret_cast<const int32_t*>(p + sz[0] + sz[1] + sz[2] + sz[3]);
  t.out_keys = reinterpret_cast<uint32_t*>(p + sz[0] + sz[1] + sz[2]);
  t.out_toks = reinterpret_cast<int32_t*>(p + sz[0] + sz[1] + sz[2] + sz[3]);
  t.idx = idx; t.cnt = cnt;
  t.Lpad = a.Lpad; t.L = a.L; t.N = budget;
  tok_plan(k, budget, t.P);
  const int rows = (int)(q.B * q.H);
  // pass 1: 256 threads x 16 tokens per part; pass 2: 16 candidates per thread, 256 or 1024 threads
  hipLaunchKernelGGL((token_topk_kernel<256, kTokPart / 256, true>), dim3(t.P, rows), dim3(256), 0, s, t);
  if (t.P * t.N <= 4096)
    hipLaunchKernelGGL((token_topk_kernel<256, 16, false>), dim3(1, rows), dim3(256), 0, s, t);
  else
    hipLaunchKernelGGL((token_topk_kernel<1024, kTokMaxCand / 1024, false>), dim3(1, rows), dim3(1024), 0, s, t);
}

}  // namespace bsa
