// Device helpers shared by the gfx950 kernels of libbsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even, with the hardware conversion (v_cvt_pk_bf16_f32; the
// bit-twiddling form compiles to a branch per element around its NaN case)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Load 8 consecutive elements (bf16 or f32) as floats.  p is 16-byte aligned.
template <int DT>
__device__ __forceinline__ void load8(const void* p, float (&o)[8]) {
  if constexpr (DT == BSA_BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16lo(w[i]); o[2 * i + 1] = bf16hi(w[i]); }
  } else {
    f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
  }
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, wave_xor(v, m));
  return v;
}
// fixed butterfly order: every lane ends with the same bits
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += wave_xor(v, m);
  return v;
}

// Wavefront reductions through DPP (no LDS round trips): quad swaps, row
// mirrors, then the row broadcasts fold the four 16-lane rows into lane 63,
// whose value is read back as a scalar.  Fixed order: identical bits in every
// lane.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __uint_as_float(dpp_u32<CTRL, ROWMASK>(__float_as_uint(old), __float_as_uint(v)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(0.f, v);          // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(0.f, v);          // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(0.f, v);         // row_half_mirror
  v += dpp_f32<0x140>(0.f, v);         // row_mirror
  v += dpp_f32<0x142, 0xa>(0.f, v);    // row_bcast:15 into rows 1, 3
  v += dpp_f32<0x143, 0xc>(0.f, v);    // row_bcast:31 into rows 2, 3
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
// wave_sum_dpp / wave_max_dpp of N independent values, stage by stage: the same
// bits as N separate calls, with the DPP latencies of the values overlapping.
template <int N>
__device__ __forceinline__ void wave_sum_dpp_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0xB1>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x4E>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x141>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x140>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x142, 0xa>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<0x143, 0xc>(0.f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v[i]), 63));
}
template <int N>
__device__ __forceinline__ void wave_max_dpp_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0xB1>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0x4E>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0x141>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0x140>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0x142, 0xa>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<0x143, 0xc>(-INFINITY, v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v[i]), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x4E>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x141>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x140>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(-INFINITY, v));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
// Inclusive prefix sum over the lanes (Hillis-Steele inside each 16-lane row
// with row shifts, then the row broadcasts carry the row totals).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += dpp_u32<0x111>(0u, v);          // row_shr:1
  v += dpp_u32<0x112>(0u, v);          // row_shr:2
  v += dpp_u32<0x114>(0u, v);          // row_shr:4
  v += dpp_u32<0x118>(0u, v);          // row_shr:8
  v += dpp_u32<0x142, 0xa>(0u, v);     // row_bcast:15 into rows 1, 3
  v += dpp_u32<0x143, 0xc>(0u, v);     // row_bcast:31 into rows 2, 3
  return v;
}

// Wavefront-wide (key, idx) with the largest key, the smallest idx among
// equal keys; the result is uniform.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ void argmax_step(uint32_t& k, uint32_t& i) {
  const uint32_t ok = dpp_u32<CTRL, ROWMASK>(0u, k), oi = dpp_u32<CTRL, ROWMASK>(0xFFFFFFFFu, i);
  const bool better = ok > k || (ok == k && oi < i);
  k = better ? ok : k;
  i = better ? oi : i;
}
__device__ __forceinline__ void wave_argmax_dpp(uint32_t& k, uint32_t& i) {
  argmax_step<0xB1>(k, i);
  argmax_step<0x4E>(k, i);
  argmax_step<0x141>(k, i);
  argmax_step<0x140>(k, i);
  argmax_step<0x142, 0xa>(k, i);
  argmax_step<0x143, 0xc>(k, i);
  k = __builtin_amdgcn_readlane(k, 63);
  i = __builtin_amdgcn_readlane(i, 63);
}

// The values of lanes l % 32 and l % 32 + 32 (gfx950 v_permlane32_swap: one
// instruction, no LDS round trip): {v[l & 31], v[(l & 31) + 32]} on every lane.
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// The values of lanes l with bit 4 clear and set (v_permlane16_swap):
// {v[l & ~16], v[l | 16]} on every lane.
__device__ __forceinline__ void lane_pair16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// Sum / max over the lanes l ^ (N * k): across the N-lane groups, lane by
// lane (N = 16: the four 16-lane rows; N = 8: the eight 8-lane groups); the
// same bits on every lane of such a set.
template <int N>
__device__ __forceinline__ float groups_sum(float v) {
  static_assert(N == 8 || N == 16, "group width");
  float lo, hi;
  if (N == 8) v += dpp_f32<0x128>(0.f, v);         // row_ror:8: lane i reads lane i ^ 8
  lane_pair16(v, lo, hi);
  v = lo + hi;
  lane_pair(v, lo, hi);
  return lo + hi;
}
template <int N>
__device__ __forceinline__ float groups_max(float v) {
  static_assert(N == 8 || N == 16, "group width");
  float lo, hi;
  if (N == 8) v = fmaxf(v, dpp_f32<0x128>(-INFINITY, v));
  lane_pair16(v, lo, hi);
  v = fmaxf(lo, hi);
  lane_pair(v, lo, hi);
  return fmaxf(lo, hi);
}
// Sum inside each N-lane group (N = 8 or 16) by DPP butterflies; the same
// bits on every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group width");
  v += dpp_f32<0xB1>(0.f, v);          // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(0.f, v);          // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(0.f, v);         // row_half_mirror
  if (N == 16) v += dpp_f32<0x140>(0.f, v);   // row_mirror
  return v;
}

// Sum over the lane pair (l, l ^ 32), the same bits on both lanes.
__device__ __forceinline__ float pair_sum(float v) {
  float lo, hi;
  lane_pair(v, lo, hi);
  return lo + hi;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Which half of the frequency chunks a head dim belongs to: 0 = fast band
// (FC index < D/4, high frequency), 1 = slow band.
__device__ __forceinline__ int band_of_dim(int d, int D, int layout) {
  int fc = (layout == BSA_ROPE_HALF) ? (d < D / 2 ? d : d - D / 2) : (d >> 1);
  return fc < D / 4 ? 0 : 1;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace bsa
