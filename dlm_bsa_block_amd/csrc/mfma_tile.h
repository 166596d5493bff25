// Building blocks of the bf16 MFMA attention tiles (gfx950).
//
// Layout of one wave's work (32 query vectors, a KV tile of KVB keys, D = 128):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16, K as the A operand (rows =
//   keys, read from LDS), Q^T as the B operand (held in registers).  Lane l
//   then owns query l % 32 and 16 keys per 32-key sub-tile:
//       key = 32*kt + 8*(i/4) + 4*(l/32) + (i%4),   i = 0..15.
//   O^T = V^T P^T with V^T as the A operand and P^T as the B operand taken
//   straight from the lane's S registers.  The gfx950 transposing LDS read
//   (ds_read_b64_tr_b16) hands each lane four consecutive keys of one head
//   dim: within a 16-lane group it returns to lane o element (o & 3) of the
//   8-byte pieces addressed by lanes (o >> 2) + 4t, t = 0..3, so lane i of the
//   group points at V[key0 + (i >> 2)][d0 + 4 (i & 3)] and lane o receives
//   V[key0 + t][d0 + o].  The key order inside each 16-key step is permuted
//   identically on both operands, so no data moves between lanes.  The output
//   O^T leaves lane l with query l % 32 and dims 32*dt + 8*(i/4) + 4*(l/32) + (i%4).
// Every per-query statistic (running max, sum) is lane-local up to the pair
// (l, l ^ 32) that shares a query.
//
// LDS tile layout (K and V alike): row r of a tile takes 256 contiguous bytes
// and its 16-byte chunk c (dims 8c .. 8c+7) sits at chunk slot c ^ swz(r),
// swz(r) = ((r & 3) << 2) | ((r >> 2) & 3).  The K reads (16 consecutive rows,
// one chunk) and the transposing V reads (4 consecutive rows, 4 consecutive
// chunks) then hit 64 distinct banks.  Tiles are filled by direct global->LDS
// copies (global_load_lds_dwordx4): one wave instruction writes 1 KB of
// consecutive LDS, i.e. four rows, each lane fetching the chunk that belongs
// in its slot.
#pragma once
#include "common.h"

namespace bsa {

constexpr int kD = 128;
constexpr int kRow = kD;                          // LDS row length in elements (no padding; swizzled)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave instruction of a direct global->LDS copy: each lane fetches 16
// bytes from its own address and the wave writes them to 1 KB of consecutive
// LDS starting at the wave-uniform byte address `lds`.  Written as inline asm
// on purpose: the compiler would otherwise treat every later LDS read as
// possibly overlapping the copy and wait for all copies in flight before it,
// which defeats the double buffering.  The copies carry no result registers;
// their completion is awaited explicitly (wait_loads_but) before a barrier.
// M0 holds the LDS address (the compiler loads it); one wait state separates
// its write from the copy.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// Same with a uniform 64-bit base and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_sv(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Start the copy of rows [0, KVB) of one K or V tile into LDS at byte address dst.  Source rows at
// or beyond nk repeat row nk - 1 (nk >= 1): they hold finite values that the
// caller masks (K) or weights by zero (V).  NW waves share the work (KVB / (4
// NW) instructions each); the copy completes asynchronously (vmcnt) and needs
// a wait plus a barrier before other waves read it.
template <int KVB, int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ src, int64_t sl, int nk, uint32_t dst) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int IT = KVB / 4 / NW;                // wave instructions per tile
  static_assert(IT * 4 * NW == KVB, "tile rows must split evenly over the waves");
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(dst);
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int m = i * NW + w;                     // this instruction fills LDS rows 4m .. 4m+3
    const int r = 4 * m + (lane >> 4);
    const int c = (lane & 15) ^ swz(r);
    const int sr = min(r, nk - 1);
    dma16(src + (int64_t)sr * sl + 8 * c, l0 + 4 * m * kRow * 2);
  }
}

// Byte offset, from the tile's first row, of the 16-byte piece this lane
// copies in every wave instruction of a whole-tile copy (issue_full_tile):
// LDS row 4 * (i * NW + w) + (lane >> 4) has the same swizzle for every i.
template <int NW>
__device__ __forceinline__ uint32_t tile_lane_offset(int64_t sl) {
  static_assert(NW % 4 == 0, "row swizzle must repeat across instructions");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = 4 * w + (lane >> 4);
  const int c = (lane & 15) ^ swz(r);
  return (uint32_t)((int64_t)r * sl * 2 + 16 * c);
}

// Copy of a whole tile (all KVB rows inside the sequence): the row step of
// each instruction is uniform, the lane's part is the fixed offset voff.
template <int KVB, int NW>
__device__ __forceinline__ void issue_full_tile(const uint16_t* __restrict__ src, int64_t sl, uint32_t voff,
                                                uint32_t dst) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int IT = KVB / 4 / NW;
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(dst);
#pragma unroll
  for (int i = 0; i < IT; ++i)
    dma16_sv(src + (int64_t)(4 * NW * i) * sl, voff, l0 + 4 * (i * NW + w) * kRow * 2);
}

__device__ __forceinline__ void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every tile copy in flight).  Callers order the copies themselves
// with wait_loads_but; the LDS reads of this wave are drained first so that a
// buffer may be overwritten once every wave has passed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}
// Wait until at most N of this wave's memory loads are still in flight.
template <int N>
__device__ __forceinline__ void wait_loads_but() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Per-lane LDS offsets (elements) of the K-operand chunks: kofs[st] for k-step st.
__device__ __forceinline__ void k_offsets(int (&kofs)[8]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hi = lane >> 5, sw = swz(r);
#pragma unroll
  for (int st = 0; st < 8; ++st) kofs[st] = r * kRow + 8 * ((2 * st + hi) ^ sw);
}

// Per-lane LDS offsets (elements) of the transposing V reads: vofs[2*dt + up]
// for dims 32*dt.. and key half up (keys +0..3 or +8..11 of each 16-key step).
__device__ __forceinline__ void v_offsets(int (&vofs)[8]) {
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5, gi = lane & 15, dgrp = (lane >> 4) & 1;
  const int rr = gi >> 2;                         // row within the 4-row group
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int up = 0; up < 2; ++up) {
      const int row = 4 * hi + 8 * up + rr;       // row offset inside the 16-key step
      const int c = 4 * dt + 2 * dgrp + ((gi & 3) >> 1);
      vofs[2 * dt + up] = row * kRow + 8 * (c ^ swz(row)) + 4 * (gi & 1);
    }
}

// Scheduling hints: keep the LDS reads of the next k-step ahead of the MFMAs
// of the current one (the compiler would otherwise issue them just in time
// and expose the LDS latency on every product).
#define BSA_SCHED_DS_READ(n) __builtin_amdgcn_sched_group_barrier(0x100, n, 0)
#define BSA_SCHED_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, n, 0)
#define BSA_SCHED_VALU(n) __builtin_amdgcn_sched_group_barrier(0x002, n, 0)

// S^T sub-tiles for one wave: s[kt] (16 floats per lane) for keys 32*kt.. of
// the tile.  With PREFETCH the K fragments of k-step st + 1 are read while
// the four products of k-step st run (32 more registers); without it the
// compiler schedules the reads itself.
template <int KVB, bool PREFETCH = true>
__device__ __forceinline__ void qk_tile(const uint16_t* Ks, const int (&kofs)[8], const bf16x8 (&qf)[8],
                                        f32x16 (&s)[KVB / 32]) {
  constexpr int NT = KVB / 32;
  if (!PREFETCH) {
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) s[kt] = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + 32 * kt * kRow + kofs[st]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kt], 0, 0, 0);
      }
    return;
  }
  bf16x8 kf[2][NT];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt) {
    s[kt] = f32x16{};
    kf[0][kt] = *reinterpret_cast<const bf16x8*>(Ks + 32 * kt * kRow + kofs[0]);
  }
  BSA_SCHED_DS_READ(NT);
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    if (st + 1 < 8) {
#pragma unroll
      for (int kt = 0; kt < NT; ++kt)
        kf[(st + 1) & 1][kt] = *reinterpret_cast<const bf16x8*>(Ks + 32 * kt * kRow + kofs[st + 1]);
      BSA_SCHED_DS_READ(NT);
    }
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st & 1][kt], qf[st], s[kt], 0, 0, 0);
    BSA_SCHED_MFMA(NT);
  }
}

// O^T += V^T P^T for one wave; p[kt] holds probabilities in the S^T layout.
template <int KVB>
__device__ __forceinline__ void pv_tile(const uint16_t* Vs, const int (&vofs)[8], const f32x16 (&p)[KVB / 32],
                                        f32x16 (&o)[4]) {
#pragma unroll
  for (int k = 0; k < KVB / 16; ++k) {
    const int kt = k >> 1, hs = k & 1;
    float f[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = p[kt][8 * hs + t];
    const bf16x8 b = pack_bf16x8(f);
    const uint16_t* step = Vs + 16 * k * kRow;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(step + vofs[2 * dt]));
      const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(step + vofs[2 * dt + 1]));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[dt], 0, 0, 0);
    }
  }
}

// Mask every S element whose key offset within the tile exceeds `lim` (lim < 0
// masks the whole tile).  Branch-free: one compare (against a literal) and
// select per element.
template <int NT>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NT], int lim) {
  const int hi = (threadIdx.x & 63) >> 5;
  const int l2 = lim - 4 * hi;                    // key offset = 32 kt + 8 (i / 4) + 4 hi + i % 4
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kt][i] = (32 * kt + 8 * (i >> 2) + (i & 3)) <= l2 ? s[kt][i] : -INFINITY;
}

// max(a, b, c) in one instruction.  Written out because fmaxf makes the
// compiler quiet every operand first (one extra instruction per element);
// the S values here are never NaN.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Largest S element of the query shared by lanes l and l ^ 32: a tree of
// three-way maxima (depth 4 for a 128-key tile).
template <int NT>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NT]) {
  constexpr int N = 16 * NT;
  float x[N];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) x[16 * kt + i] = s[kt][i];
  int n = N;
#pragma unroll
  for (int lvl = 0; lvl < 6; ++lvl) {
    if (n > 1) {
      const int m = n / 3, r = n - 3 * m;
#pragma unroll
      for (int j = 0; j < m; ++j) x[j] = max3f(x[3 * j], x[3 * j + 1], x[3 * j + 2]);
      if (r == 1) x[m] = x[3 * m];
      if (r == 2) x[m] = max3f(x[3 * m], x[3 * m + 1], x[3 * m + 1]);
      n = m + (r ? 1 : 0);
    }
  }
  float lo, hi;
  lane_pair(x[0], lo, hi);
  return max3f(lo, hi, hi);
}

// Online-softmax bookkeeping for one tile, in log2 units.  m_ref is the
// running max; O and l are rescaled only when some query of the wave sees a
// larger tile maximum tm2 (a wave-uniform branch), otherwise the 64
// multiplies are skipped.  The reference is never left below the running
// max: then the largest probability is exactly 1, which bf16 holds without
// rounding, and the dominant term of P V carries no rounding of P (a stale
// reference lets that term carry a 2^-9 relative error straight into the
// output).  Returns the offset to subtract from s * c2.
__device__ __forceinline__ float softmax_rescale(float tm2, float& m_ref, float& l_run, f32x16 (&o)[4]) {
  if (__builtin_amdgcn_ballot_w64(tm2 > m_ref) != 0ull) {
    const float m_new = fmaxf(m_ref, tm2);
    const float alpha = fast_exp2(m_ref - (m_new == -INFINITY ? 0.f : m_new));
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    m_ref = m_new;
  }
  return m_ref == -INFINITY ? 0.f : m_ref;
}

// s <- p = 2^(s c2 - msub) for the whole tile; adds the lane's part of the
// row sum to l_run.
template <int NT>
__device__ __forceinline__ void softmax_probs(f32x16 (&s)[NT], float c2, float msub, float& l_run) {
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[kt][i] = fast_exp2(fmaf(s[kt][i], c2, -msub));
      part[i & 3] += s[kt][i];
    }
  l_run += (part[0] + part[1]) + (part[2] + part[3]);
}

// p = 2^(s c2 - msub) and O^T += V^T P^T for one wave, one 16-key step at a
// time: the exponentials of step k + 1 (vector ALU) run while the four
// products of step k occupy the matrix core, and the transposing V reads of
// step k + 1 are issued ahead of them.  Adds the lane's part of the row sum
// of p to l_run.
template <int KVB>
__device__ __forceinline__ void softmax_pv_tile(const uint16_t* Vs, const int (&vofs)[8], const f32x16 (&s)[KVB / 32],
                                                float c2, float msub, float& l_run, f32x16 (&o)[4]) {
  constexpr int NS = KVB / 16;                    // 16-key steps
  const uint16_t* vb[8];                          // per-lane read bases; the step is an immediate offset
#pragma unroll
  for (int x = 0; x < 8; ++x) vb[x] = Vs + vofs[x];
  v4i16 vf[2][8];
  auto read_step = [&](int k, v4i16 (&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
      dst[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb[x] + 16 * k * kRow));
  };
  auto probs = [&](int k) __attribute__((always_inline)) {
    const int kt = k >> 1, hs = k & 1;
    float f[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = fast_exp2(fmaf(s[kt][8 * hs + t], c2, -msub));
    l_run += ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
    return pack_bf16x8(f);
  };
  read_step(0, vf[0]);
  bf16x8 b = probs(0);
  BSA_SCHED_DS_READ(8);
  BSA_SCHED_VALU(32);
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (k + 1 < NS) {
      read_step(k + 1, vf[(k + 1) & 1]);
      BSA_SCHED_DS_READ(8);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(vf[k & 1][2 * dt], vf[k & 1][2 * dt + 1], 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[dt], 0, 0, 0);
    }
    if (k + 1 < NS) {
      b = probs(k + 1);
      // one product, then a share of the next step's exponentials, ...
      BSA_SCHED_MFMA(1);
      BSA_SCHED_VALU(8);
      BSA_SCHED_MFMA(1);
      BSA_SCHED_VALU(8);
      BSA_SCHED_MFMA(1);
      BSA_SCHED_VALU(8);
      BSA_SCHED_MFMA(1);
      BSA_SCHED_VALU(8);
    } else {
      BSA_SCHED_MFMA(4);
    }
  }
}

// key offset (within the tile) of S element i of sub-tile kt held by this lane
__device__ __forceinline__ int s_key(int kt, int i) {
  const int hi = (threadIdx.x & 63) >> 5;
  return 32 * kt + 8 * (i >> 2) + 4 * hi + (i & 3);
}

// dim of O element i of sub-tile dt held by this lane
__device__ __forceinline__ int o_dim(int dt, int i) {
  const int hi = (threadIdx.x & 63) >> 5;
  return 32 * dt + 8 * (i >> 2) + 4 * hi + (i & 3);
}

// Store the lane's part of one normalised output row, O^T tiles o scaled by
// inv: element 4 i4 + e of tile dt is dim 32 dt + 8 i4 + 4 hi + e.  The row
// is bf16 (rounded to nearest even) or f32.
__device__ __forceinline__ void store_o_row(void* orow, bool f32, const f32x16 (&o)[4], float inv, int hi) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * dt + 8 * i4 + 4 * hi;
      const float a = o[dt][4 * i4] * inv, b = o[dt][4 * i4 + 1] * inv;
      const float c = o[dt][4 * i4 + 2] * inv, e = o[dt][4 * i4 + 3] * inv;
      if (f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(orow) + d) = f32x4{a, b, c, e};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(orow) + d) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, e)};
      }
    }
}

// Make the compiler wait here for the loads that filled qf (an empty asm
// that reads them), so that it need not wait for them later, when tile
// copies it cannot see are in flight behind them.
__device__ __forceinline__ void settle(bf16x8 (&qf)[8]) {
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" ::"v"(qf[st]));
}

// Load the lane's Q^T operand fragments: query row pointer (bf16, D = 128).
// The loads of load_q_frag alone (qrow readable); zero_q_frag applies the
// validity afterwards, where the fragments are first needed.
__device__ __forceinline__ void load_q_frag_raw(const uint16_t* qrow, bf16x8 (&qf)[8]) {
  const int hi = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int st = 0; st < 8; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hi);
}
__device__ __forceinline__ void zero_q_frag(bool valid, bf16x8 (&qf)[8]) {
#pragma unroll
  for (int st = 0; st < 8; ++st) qf[st] = valid ? qf[st] : bf16x8{};
}

// qrow must be a readable row (callers clamp it); a lane with valid = false gets
// zeros.  The loads are made whatever valid is (a load under a branch would
// make the compiler wait for it where the branch joins).
__device__ __forceinline__ void load_q_frag(const uint16_t* qrow, bool valid, bf16x8 (&qf)[8]) {
  const int hi = (threadIdx.x & 63) >> 5;
  u32x4 w[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) w[st] = *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * hi);
#pragma unroll
  for (int st = 0; st < 8; ++st) qf[st] = __builtin_bit_cast(bf16x8, valid ? w[st] : u32x4{0, 0, 0, 0});
}

}  // namespace bsa
