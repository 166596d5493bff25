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
//      K of the slice streams through (eight 16-key passes of loads in flight
//      per thread), q.k for the G heads of the group (log2 units) and each
//      tile's max go to the workspace;
//   2. pv_kernel: same grid; the max over all newer slices' tiles seeds the
//      walk of the slice's own tiles, which decides every (head, tile); V is
//      loaded only for tiles some head keeps (the G heads share each load,
//      NSA implementation-challenges section), and each head accumulates
//      2^(s - m_s) v over its kept tiles, m_s being its largest kept tile max
//      in the slice;
//   3. the combine kernel merges the slices' (m, l, o) in order.
#include "common.cuh"
#include "internal.h"
#include "split.h"

namespace bsa {

constexpr int kTDecTile = 64;           // keys per tile
constexpr int kTDecMaxSplit = 2048;     // keys per slice, at most
constexpr int kTDecPass = 16;           // keys per workgroup pass (4 waves x 4 keys)
constexpr int kTDecBatch = 8;           // passes whose loads are in flight together

struct TDecArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t qsb, qsh, ksb, ksh, ksl, vsb, vsh, vsl;
  int Hkv, L, Lpad, split, nsplit, ntiles;
  float c2;                             // scale * log2(e)
  float ln_lam2;                        // ln(lambda) * log2(e); -inf for lambda = 0
  float* scores;                        // [B][Hkv][G][Lpad], log2 units; Lpad = L rounded up to 4
  float* tmax;                          // [B][Hkv][G][ntiles]
  float* smax;                          // [B][Hkv][G][nsplit] max over a slice's tiles
  float* part_o;                        // [B][Hkv][nsplit][G][D]
  float* part_ml;                       // [B][Hkv][nsplit][G][2]
  int32_t* kept;                        // [B][Hq] kept tiles per head, or null
  uint8_t* keep_map;                    // [B][Hq][ntiles] or null
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
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v4 = {0u, 0u, 0u, 0u};
    if (col < G)
      v4 = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.qsb + (int64_t)(g * G + col) * a.qsh +
                                                  32 * ks + 8 * kq) * 2);
    qb[ks] = __builtin_bit_cast(bf16x8, v4);
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
    if (split == 0 && a.kept) a.kept[hb + tid] = 0;   // the decision kernel adds every slice's count
  }
}

// Decisions, V and P V of one slice, eight waves.  Round trip one brings the
// slice's scores (into LDS, key-major), its tile maxima and the maxima of all
// newer slices; every wave then takes the decisions of all (head, tile) pairs
// itself -- tile j of head h is kept iff its max tm passes the test against
// the max of every newer tile -- and issues its V loads at once.  The waves
// split the head dims (16 each, 4 lanes x 4 dims per key row, 16 keys per
// pass), so every wave walks all kept tiles of the slice (the G heads share
// each V load) and the work stays even however few tiles are kept.  While the
// loads are in flight the workgroup turns the kept scores into
// p = 2^(s - m_s) in place (m_s: the head's largest kept tile max in the
// slice; 0 for a tile or key the head does not keep).
template <int G>
__global__ __launch_bounds__(512, G == 8 ? 2 : 4) void tdec_pv_kernel(TDecArgs a) {
  constexpr int D = 128, T = kTDecTile, NW = 8, NT = 512;
  constexpr int MAXT = kTDecMaxSplit / T;           // 32 tiles per slice at most
  constexpr int NPAIR = (2 * G + 3) / 4;            // ballots of (head, tile) pairs: 2 heads x 32 tiles each
  constexpr int DW = D / NW, LPK = DW / 4;          // dims per wave, lanes per key row
  constexpr int KPP = 64 / LPK, PPT = T / KPP;      // keys per pass, passes per tile
  constexpr int CH = 8;                             // kept tiles whose loads are in flight together
  constexpr int TPI = NT / (T * G);                 // tiles per step of the p pass
  static_assert(TPI >= 1, "one tile of (key, head) pairs per step at most");
  __shared__ __align__(16) float sc[kTDecMaxSplit * G];   // [key][head]: scores, then p
  __shared__ float tmx[G][MAXT];
  __shared__ float newer_sh[G];

  const int split = a.nsplit - 1 - (int)blockIdx.x;         // newest slices (most kept tiles) first
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int s0 = split * a.split;
  const int n = min(a.split, a.L - s0);
  const int nt = (n + T - 1) / T;
  const int nq = (n + 3) / 4;                               // 16-byte score chunks per head row
  const int64_t hb = ((int64_t)b * a.Hkv + g) * G;

  // ---- round trip 1
  {
    f32x4 sv[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const int i = min(tid + NT * r, G * nq - 1);
      const int h = i / nq, c = i - h * nq;
      sv[r] = *reinterpret_cast<const f32x4*>(a.scores + (hb + h) * a.Lpad + s0 + 4 * c);
    }
    float tv = -INFINITY;
    if (tid < G * MAXT) {
      const int h = tid / MAXT, j = tid - h * MAXT;
      if (j < nt) tv = a.tmax[(hb + h) * a.ntiles + s0 / T + j];
    }
    float nv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      nv[h] = -INFINITY;
      if (w == NW - 1)
        for (int sp = split + 1 + lane; sp < a.nsplit; sp += 64) nv[h] = fmaxf(nv[h], a.smax[(hb + h) * a.nsplit + sp]);
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const int i = tid + NT * r;
      if (i < G * nq) {
        const int h = i / nq, c = i - h * nq;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[(4 * c + e) * G + h] = sv[r][e];
      }
    }
    if (tid < G * MAXT) tmx[tid / MAXT][tid % MAXT] = tv;
    if (w == NW - 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m = wave_max_dpp(nv[h]);
        if (lane == 0) newer_sh[h] = m;
      }
    }
  }
  __syncthreads();

  // ---- decisions: ballot r covers heads 2r (lanes 0-31) and 2r + 1 (lanes 32-63), lane % 32 = tile
  uint32_t kb[G];
  float mk[G];
  uint32_t any = 0u;
#pragma unroll
  for (int r = 0; r < NPAIR; ++r) {
    const int h = 2 * r + lane / 32, j = lane % 32;
    const bool valid = h < G && j < nt;
    const float tm = valid ? tmx[h < G ? h : 0][j] : -INFINITY;
    // max over tiles j' > j of the slice (shuffles stay inside each 32-lane half)
    float incl = tm;
#pragma unroll
    for (int sft = 1; sft < 32; sft <<= 1) incl = fmaxf(incl, __shfl_down(incl, sft, 32));
    float excl = __shfl_down(incl, 1, 32);
    if (j == 31) excl = -INFINITY;
    const float M = fmaxf(valid ? newer_sh[h] : -INFINITY, excl);
    const bool keep = valid && tm > -INFINITY && (M == -INFINITY || tm - M >= a.ln_lam2);
    const uint64_t bal = __ballot(keep);
    float x = keep ? tm : -INFINITY;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 32));
    const float x0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 0));
    const float x1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 32));
    if (2 * r < G) { kb[2 * r] = (uint32_t)bal; mk[2 * r] = x0; any |= (uint32_t)bal; }
    if (2 * r + 1 < G) { kb[2 * r + 1] = (uint32_t)(bal >> 32); mk[2 * r + 1] = x1; any |= (uint32_t)(bal >> 32); }
    if (w == 0 && valid && a.keep_map) a.keep_map[(hb + h) * a.ntiles + s0 / T + j] = keep ? 1 : 0;
  }
  float msub[G];
#pragma unroll
  for (int h = 0; h < G; ++h) msub[h] = mk[h] == -INFINITY ? 0.f : mk[h];
  if (w == 0 && lane < G && a.kept) {
    uint32_t c = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) if (lane == h) c = __popc(kb[h]);
    atomicAdd(a.kept + hb + lane, (int)c);
  }

  // ---- V of the kept tiles (CH at a time), p in place, P V
  const int kw = lane / LPK, dl = w * DW + (lane % LPK) * 4;   // key row of the pass, first dim
  // uniform base of the slice's V rows, 32-bit lane offsets (the host bounds kv_split rows of stride vsl)
  const uint8_t* vb = a.v + ((int64_t)b * a.vsb + (int64_t)g * a.vsh + (int64_t)s0 * a.vsl) * 2;
  const uint32_t rowb = (uint32_t)a.vsl * 2u;
  float acc[G][4], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
  }
  uint32_t todo = any;
  bool pdone = false;
  while (todo) {                                     // the same on every wave
    int tl[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      tl[c] = todo ? __builtin_ctz(todo) : -1;
      todo &= todo - 1u;
    }
    u32x2 vv[CH][PPT];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (tl[c] < 0) continue;
#pragma unroll
      for (int p = 0; p < PPT; ++p) {
        const uint32_t kr = (uint32_t)min(tl[c] * T + KPP * p + kw, n - 1);
        vv[c][p] = *reinterpret_cast<const u32x2*>(vb + (kr * rowb + (uint32_t)dl * 2u));
      }
    }
    if (!pdone) {
      // p for every (key, head) of every kept tile, keys past the slice included (p = 0)
      const int ts = tid / (T * G), ke = tid % (T * G);
      const int h = ke % G;
      uint32_t kbh = 0u;
      float ms = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        if (hh == h) { kbh = kb[hh]; ms = msub[hh]; }
      for (int t0 = 0; t0 < nt; t0 += TPI) {
        const int t = t0 + ts;
        if (t < nt && ((any >> t) & 1u)) {
          const int key = t * T + ke / G;
          float* ps = &sc[key * G + h];
          const bool use = ((kbh >> t) & 1u) && key < n;
          *ps = use ? fast_exp2(*ps - ms) : 0.f;
        }
      }
      __syncthreads();
      pdone = true;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (tl[c] < 0) continue;
#pragma unroll
      for (int p = 0; p < PPT; ++p) {
        const int key = tl[c] * T + KPP * p + kw;
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

  // ---- sums over the 16 key rows of the wave; each wave owns its dims
  const int64_t pbase = (((int64_t)b * a.Hkv + g) * a.nsplit + split) * G;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = acc[h][e];
      x += dpp_f32<0x124>(0.f, x);                  // row_ror:4
      x += dpp_f32<0x128>(0.f, x);                  // row_ror:8
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
      }
    }
  }
}

static size_t tdec_sizes(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t (&sz)[5]) {
  const int64_t nsplit = ceil_div(k.L, kv_split), ntiles = ceil_div(k.L, kTDecTile);
  const size_t heads = (size_t)q.B * q.H;            // B * Hkv * G
  const size_t n = heads * nsplit;
  sz[0] = align256(heads * ((k.L + 3) & ~3LL) * 4);    // scores, rows padded to 16 bytes
  sz[1] = align256(heads * ntiles * 4);                // tile maxima
  sz[2] = align256(n * q.D * 4);                       // partial O
  sz[3] = align256(n * 2 * 4);                         // partial (m, l)
  sz[4] = align256(n * 4);                             // slice maxima
  return sz[0] + sz[1] + sz[2] + sz[3] + sz[4];
}

bool plan_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t& bytes) {
  size_t sz[5];
  bytes = tdec_sizes(q, k, kv_split, sz);
  return true;
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
  a.Hkv = (int)k.H; a.L = (int)k.L; a.Lpad = (int)((k.L + 3) & ~3LL); a.split = kv_split;
  a.nsplit = (int)ceil_div(k.L, kv_split);
  a.ntiles = (int)ceil_div(k.L, kTDecTile);
  a.c2 = scale * kLog2e;
  a.ln_lam2 = lambda > 0.f ? logf(lambda) * kLog2e : -INFINITY;
  size_t sz[5];
  tdec_sizes(q, k, kv_split, sz);
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.scores = reinterpret_cast<float*>(p);
  a.tmax = reinterpret_cast<float*>(p + sz[0]);
  a.part_o = reinterpret_cast<float*>(p + sz[0] + sz[1]);
  a.part_ml = reinterpret_cast<float*>(p + sz[0] + sz[1] + sz[2]);
  a.smax = reinterpret_cast<float*>(p + sz[0] + sz[1] + sz[2] + sz[3]);
  a.kept = kept;
  a.keep_map = keep_map;
  dim3 grid(a.nsplit, q.B * k.H);
#define BSA_TDEC(GG)                                                                  \
  hipLaunchKernelGGL(tdec_scores_kernel<GG>, grid, dim3(512), 0, s, a);               \
  hipLaunchKernelGGL(tdec_pv_kernel<GG>, grid, dim3(512), 0, s, a)
  switch (G) {
    case 1: BSA_TDEC(1); break;
    case 2: BSA_TDEC(2); break;
    case 4: BSA_TDEC(4); break;
    default: BSA_TDEC(8); break;
  }
#undef BSA_TDEC
  CombArgs c;
  c.part_o = a.part_o; c.part_ml = a.part_ml; c.cnt = nullptr; c.items = a.nsplit;
  c.unit_num = 1; c.unit_den = 1;
  c.qvc = 256 / (int)q.D;
  c.Hkv = (int)k.H; c.G = G; c.NQB = 1; c.q_block = 1; c.Lq = 1; c.D = (int)q.D; c.QV = G;
  c.row_mask = nullptr; c.o = o.data; c.osb = o.stride_b; c.osh = o.stride_h; c.osl = o.stride_l; c.lse = lse;
  launch_combine(c, o.dtype, (int)q.B, s);
}

}  // namespace bsa
