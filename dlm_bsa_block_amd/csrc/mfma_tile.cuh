// Building blocks of the bf16 MFMA attention tiles (gfx950).
//
// Layout of one wave's work (32 query vectors, a KV tile of KVB keys, D = 128):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16, K as the A operand (rows =
//   keys, read from LDS), Q^T as the B operand (held in registers).  Lane l
//   then owns query l % 32 and 16 keys per 32-key sub-tile:
//       key = 32*kt + 8*(i/4) + 4*(l/32) + (i%4),   i = 0..15.
//   O^T = V^T P^T with V^T as the A operand (from a transposed LDS copy of V)
//   and P^T as the B operand taken straight from the lane's S registers.  The
//   key order inside each 16-key step is permuted consistently on both
//   operands, so no data moves between lanes.  The output O^T leaves lane l
//   with query l % 32 and dims 32*dt + 8*(i/4) + 4*(l/32) + (i%4).
// Every per-query statistic (running max, sum) is lane-local up to the pair
// (l, l ^ 32) that shares a query.
#pragma once
#include "common.cuh"

namespace bsa {

constexpr int kD = 128;
constexpr int kKStride = kD + 8;                 // K tile row stride in LDS (elements)
template <int KVB> struct VtStride { static constexpr int value = KVB + 4; };

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}

// Stage a KV tile: K rows [0, nk) row-major into Ks, V transposed into Vt
// (Vt[d][key]); rows >= nk are zero.  Called by all 256 threads.
template <int KVB>
__device__ __forceinline__ void stage_kv_tile(const uint16_t* __restrict__ kbase, int64_t ksl,
                                              const uint16_t* __restrict__ vbase, int64_t vsl, int nk,
                                              uint16_t* Ks, uint16_t* Vt, bool load_k, bool load_v) {
  constexpr int VST = VtStride<KVB>::value;
  const int tid = threadIdx.x;
  if (load_k) {
    u32x4 kr[KVB / 16];
#pragma unroll
    for (int i = 0; i < KVB / 16; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
      kr[i] = row < nk ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)row * ksl + col) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < KVB / 16; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * kKStride + col) = kr[i];
    }
  }
  if (load_v) {
    constexpr int UNITS = KVB / 64;              // (4 keys x 8 dims) units per thread
    u32x4 vr[UNITS][4];
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + 256 * i, d8 = (u & 15) * 8, k0 = (u >> 4) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[i][r] = (k0 + r) < nk ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)(k0 + r) * vsl + d8)
                                 : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = tid + 256 * i, d8 = (u & 15) * 8, k0 = (u >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of each of the 4 rows -> 4 consecutive keys of dim d8 + e
        const int wsel = e >> 1, sh = (e & 1) * 16;
        const uint32_t a0 = (vr[i][0][wsel] >> sh) & 0xFFFFu, a1 = (vr[i][1][wsel] >> sh) & 0xFFFFu;
        const uint32_t a2 = (vr[i][2][wsel] >> sh) & 0xFFFFu, a3 = (vr[i][3][wsel] >> sh) & 0xFFFFu;
        u32x2 pk = {a0 | (a1 << 16), a2 | (a3 << 16)};
        *reinterpret_cast<u32x2*>(Vt + (d8 + e) * VST + k0) = pk;
      }
    }
  }
}

// S^T sub-tiles for one wave: s[kt] (16 floats per lane) for keys 32*kt.. of the tile.
template <int KVB>
__device__ __forceinline__ void qk_tile(const uint16_t* Ks, const bf16x8 (&qf)[8], f32x16 (&s)[KVB / 32]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < KVB / 32; ++kt) {
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (32 * kt + r) * kKStride + 16 * st + 8 * hi);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], acc, 0, 0, 0);
    }
    s[kt] = acc;
  }
}

// O^T += V^T P^T for one wave; p[kt] holds probabilities in the S^T layout.
template <int KVB>
__device__ __forceinline__ void pv_tile(const uint16_t* Vt, const f32x16 (&p)[KVB / 32], f32x16 (&o)[4]) {
  constexpr int VST = VtStride<KVB>::value;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < KVB / 32; ++kt) {
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      float f[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) f[t] = p[kt][8 * hs + t];
      const bf16x8 b = pack_bf16x8(f);
      const int base = 32 * kt + 16 * hs + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* row = Vt + (32 * dt + r) * VST;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row + base);
        const u32x2 up = *reinterpret_cast<const u32x2*>(row + base + 8);
        const u32x4 w = {lo[0], lo[1], up[0], up[1]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, w);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[dt], 0, 0, 0);
      }
    }
  }
}

// Mask every S element whose key offset within the tile exceeds `lim` (lim < 0
// masks the whole tile).  Branch-free: one compare and select per element.
template <int NT>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NT], int lim) {
  const int hi = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = 32 * kt + 8 * (i >> 2) + 4 * hi + (i & 3);
      s[kt][i] = kk <= lim ? s[kt][i] : -INFINITY;
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

// Load the lane's Q^T operand fragments: query row pointer (bf16, D = 128).
__device__ __forceinline__ void load_q_frag(const uint16_t* qrow, bool valid, bf16x8 (&qf)[8]) {
  const int hi = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    u32x4 w = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
    qf[st] = __builtin_bit_cast(bf16x8, w);
  }
}

}  // namespace bsa
