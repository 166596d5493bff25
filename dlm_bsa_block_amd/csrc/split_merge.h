// Split-KV partials merged inside the launch that produced them.
//
// Each workgroup publishes its slice's unnormalised partial (m, l, o) with
// device-scope stores (coherent across the XCDs' L2 caches, so no cache
// write-back or fence is needed), waits for them, and counts its arrival on the
// (row, group)'s counter.  The workgroup that counts last merges every slice in
// ascending order -- batches of 32 with a running maximum, the order of the
// separate combine -- and writes O and the natural-log LSE.  The counter is
// advanced with a wrapping increment (atomicInc with limit n - 1), so the last
// arrival returns it to zero: a counter that starts a launch at zero ends it at
// zero.
#pragma once
#include "common.h"

namespace bsa {

// Counters of the attention entry point sit in a fixed region at the front of
// its workspace, one 64-byte line each, so that calls of any shape find them
// where earlier calls left them (zero).
constexpr int kArrivalStride = 16;                                  // words per counter
constexpr int kArrivalRows = 1024;                                  // counters in the region
constexpr size_t kArrivalBytes = (size_t)kArrivalRows * kArrivalStride * 4;   // 64 KiB

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev2(float* p, float lo, float hi) {
  const uint64_t v = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const float* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of the workgroup once its device-scope partial stores
// are issued: waits for them, counts the arrival, and returns (uniformly)
// whether this workgroup was the n-th, i.e. the last, of the launch to arrive.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int n, int& flag_sh) {
  __builtin_amdgcn_s_waitcnt(0);                        // this wave's partial stores are done
  __syncthreads();                                      // ... and every wave's
  if (threadIdx.x == 0) flag_sh = (int)atomicInc(counter, (uint32_t)(n - 1)) == n - 1;
  __syncthreads();
  return flag_sh != 0;
}

// Merge of n published slices of one (row, group) by a workgroup of 256
// threads, two dims of one head per thread.  po: slice 0's partial O
// ([slice][G][D]); pml: slice 0's (m, l) ([slice][G][2], m in log2 units).
// Output: head h's O row at o + o_off + h * osh (bf16, or f32 when o_f32), its
// LSE at lse[h * lse_h].  ml_sh: LDS for G * 32 (m, l) pairs.
// Per batch of 32 slices every thread loads one (m, l) pair into LDS and its own
// dims of the 32 partial O's (at most 33 loads in flight per thread, so none
// waits for a free counter slot).
template <int G, int D>
__device__ __forceinline__ void merge_published(const float* po, const float* pml, int n, uint64_t* ml_sh, void* o,
                                                int o_f32, int64_t o_off, int64_t osh, float* lse, int64_t lse_h) {
  constexpr int BATCH = 32;
  static_assert(BATCH * G <= 256, "one (m, l) pair per thread and batch");
  constexpr int NPOS = G * D / 2;                       // (head, dim pair) positions
  constexpr int PPT = (NPOS + 255) / 256;
  const int tid = threadIdx.x;
  float M[PPT], L[PPT], acc0[PPT], acc1[PPT];
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) { M[pp] = -INFINITY; L[pp] = 0.f; acc0[pp] = 0.f; acc1[pp] = 0.f; }
  for (int it0 = 0; it0 < n; it0 += BATCH) {
    if (it0 > 0) __syncthreads();                       // the previous batch's LDS reads are done
    uint64_t mlv = 0;
    if (tid < BATCH * G) {                              // entry tid = (head, slice of the batch)
      const int h = tid / BATCH, u = tid - h * BATCH;
      const int it = min(it0 + u, n - 1);
      mlv = ld_dev_u64(pml + ((int64_t)it * G + h) * 2);
    }
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int i = tid + 256 * pp;
      // threads past the positions load a valid position too: loads under a branch would make
      // the compiler wait for each one before the next
      const int ic = min(i, NPOS - 1);
      const int h = ic / (D / 2), d = 2 * (ic - h * (D / 2));
      float o0[BATCH], o1[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int it = min(it0 + u, n - 1);
        const uint64_t ov = ld_dev_u64(po + ((int64_t)it * G + h) * D + d);
        o0[u] = __uint_as_float((uint32_t)ov);
        o1[u] = __uint_as_float((uint32_t)(ov >> 32));
      }
      if (pp == 0) {
        if (tid < BATCH * G) ml_sh[tid] = mlv;
        __syncthreads();
      }
      if (i < NPOS) {
        // this head's (m, l) of the batch, read together (16-byte LDS reads)
        uint64_t mlr[BATCH];
#pragma unroll
        for (int q = 0; q < BATCH / 2; ++q) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(&ml_sh[h * BATCH + 2 * q]);
          mlr[2 * q] = (uint64_t)t[0] | ((uint64_t)t[1] << 32);
          mlr[2 * q + 1] = (uint64_t)t[2] | ((uint64_t)t[3] << 32);
        }
        float bm = M[pp];
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (it0 + u < n) bm = fmaxf(bm, __uint_as_float((uint32_t)mlr[u]));
        if (bm == -INFINITY) continue;
        const float alpha = M[pp] == -INFINITY ? 0.f : fast_exp2(M[pp] - bm);
        L[pp] *= alpha;
        acc0[pp] *= alpha;
        acc1[pp] *= alpha;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const uint64_t ml = mlr[u];
          const float mv = __uint_as_float((uint32_t)ml);
          // selects, not a branch per slice: a slot past the count or with nothing visible keeps
          // the sums as they are (its stale values are never multiplied in)
          const bool use = it0 + u < n && mv != -INFINITY;
          const float wgt = fast_exp2(mv - bm);
          const float l2 = fmaf(__uint_as_float((uint32_t)(ml >> 32)), wgt, L[pp]);
          const float a0 = fmaf(o0[u], wgt, acc0[pp]), a1 = fmaf(o1[u], wgt, acc1[pp]);
          L[pp] = use ? l2 : L[pp];
          acc0[pp] = use ? a0 : acc0[pp];
          acc1[pp] = use ? a1 : acc1[pp];
        }
        M[pp] = bm;
      }
    }
  }
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    const int i = tid + 256 * pp;
    if (i >= NPOS) continue;
    const int h = i / (D / 2), d = 2 * (i - h * (D / 2));
    const float r0 = L[pp] > 0.f ? acc0[pp] / L[pp] : 0.f, r1 = L[pp] > 0.f ? acc1[pp] / L[pp] : 0.f;
    const int64_t oi = o_off + (int64_t)h * osh + d;
    if (o_f32) {
      static_cast<float*>(o)[oi] = r0;
      static_cast<float*>(o)[oi + 1] = r1;
    } else {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + oi) = pack_bf16x2(r0, r1);
    }
    if (d == 0) lse[(int64_t)h * lse_h] = L[pp] > 0.f ? (M[pp] + log2f(L[pp])) * kLn2 : -INFINITY;
  }
}

}  // namespace bsa
