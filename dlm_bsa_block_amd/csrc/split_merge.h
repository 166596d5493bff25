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

// Running merge state of one thread: PPT (head, dim pair) positions.
template <int G, int D>
struct MergeState {
  static constexpr int NPOS = G * D / 2;                // (head, dim pair) positions
  static constexpr int PPT = (NPOS + 255) / 256;
  float M[PPT], L[PPT], acc0[PPT], acc1[PPT];
};

// Merge of the published slices first .. first + n - 1 of one (row, group) by a
// workgroup of 256 threads, two dims of one head per thread.  po: slice 0's
// partial O ([slice][G][D]); pml: slice 0's (m, l) ([slice][G][2], m in log2
// units); ml_sh: LDS for G * 32 (m, l) pairs.  Per batch of 32 slices every
// thread loads one (m, l) pair into LDS and its own dims of the 32 partial O's
// (at most 33 loads in flight per thread, so none waits for a free counter
// slot), then merges them in ascending order with a running maximum.
template <int G, int D>
__device__ __forceinline__ void merge_run(const float* po, const float* pml, int first, int n, uint64_t* ml_sh,
                                          MergeState<G, D>& st) {
  constexpr int BATCH = 32;
  static_assert(BATCH * G <= 256, "one (m, l) pair per thread and batch");
  constexpr int NPOS = MergeState<G, D>::NPOS, PPT = MergeState<G, D>::PPT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pp = 0; pp < PPT; ++pp) {
    st.M[pp] = -INFINITY;
    st.L[pp] = 0.f;
    st.acc0[pp] = 0.f;
    st.acc1[pp] = 0.f;
  }
  for (int it0 = 0; it0 < n; it0 += BATCH) {
    __syncthreads();                                    // earlier reads of ml_sh are done
    uint64_t mlv = 0;
    if (tid < BATCH * G) {                              // entry tid = (head, slice of the batch)
      const int h = tid / BATCH, u = tid - h * BATCH;
      const int it = first + min(it0 + u, n - 1);
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
        const int it = first + min(it0 + u, n - 1);
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
        float bm = st.M[pp];
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (it0 + u < n) bm = fmaxf(bm, __uint_as_float((uint32_t)mlr[u]));
        if (bm == -INFINITY) continue;
        const float alpha = st.M[pp] == -INFINITY ? 0.f : fast_exp2(st.M[pp] - bm);
        st.L[pp] *= alpha;
        st.acc0[pp] *= alpha;
        st.acc1[pp] *= alpha;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const uint64_t ml = mlr[u];
          const float mv = __uint_as_float((uint32_t)ml);
          // selects, not a branch per slice: a slot past the count or with nothing visible keeps
          // the sums as they are (its stale values are never multiplied in)
          const bool use = it0 + u < n && mv != -INFINITY;
          const float wgt = fast_exp2(mv - bm);
          const float l2 = fmaf(__uint_as_float((uint32_t)(ml >> 32)), wgt, st.L[pp]);
          const float a0 = fmaf(o0[u], wgt, st.acc0[pp]), a1 = fmaf(o1[u], wgt, st.acc1[pp]);
          st.L[pp] = use ? l2 : st.L[pp];
          st.acc0[pp] = use ? a0 : st.acc0[pp];
          st.acc1[pp] = use ? a1 : st.acc1[pp];
        }
        st.M[pp] = bm;
      }
    }
  }
}

__device__ __forceinline__ void store_pair(void* o, int o_f32, int64_t oi, float r0, float r1) {
  if (o_f32) {
    static_cast<float*>(o)[oi] = r0;
    static_cast<float*>(o)[oi + 1] = r1;
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + oi) = pack_bf16x2(r0, r1);
  }
}

// All n published slices of one (row, group) merged; writes head h's O row at
// o + o_off + h * osh (bf16, or f32 when o_f32) and its natural-log LSE at
// lse[h * lse_h].
template <int G, int D>
__device__ __forceinline__ void merge_published(const float* po, const float* pml, int n, uint64_t* ml_sh, void* o,
                                                int o_f32, int64_t o_off, int64_t osh, float* lse, int64_t lse_h) {
  MergeState<G, D> st;
  merge_run<G, D>(po, pml, 0, n, ml_sh, st);
#pragma unroll
  for (int pp = 0; pp < MergeState<G, D>::PPT; ++pp) {
    const int i = threadIdx.x + 256 * pp;
    if (i >= MergeState<G, D>::NPOS) continue;
    const int h = i / (D / 2), d = 2 * (i - h * (D / 2));
    const float r0 = st.L[pp] > 0.f ? st.acc0[pp] / st.L[pp] : 0.f;
    const float r1 = st.L[pp] > 0.f ? st.acc1[pp] / st.L[pp] : 0.f;
    store_pair(o, o_f32, o_off + (int64_t)h * osh + d, r0, r1);
    if (d == 0) lse[(int64_t)h * lse_h] = st.L[pp] > 0.f ? (st.M[pp] + log2f(st.L[pp])) * kLn2 : -INFINITY;
  }
}

// Two runs of published slices -- the selected blocks' n_sel slices, then the
// sliding window's n_win (NSA structure section: one output per branch, mixed
// by the gates) -- merged apart and written as O = g0 O_sel + g1 O_win, with
// one natural-log LSE per branch at lse[2 h], lse[2 h + 1] (lse_h apart per
// head) and the gates at gates[2 h], gates[2 h + 1] (gate_h apart), or 1 and 1
// when gates is null.
template <int G, int D>
__device__ __forceinline__ void merge_published_window(const float* po, const float* pml, int n_sel, int n_win,
                                                       uint64_t* ml_sh, void* o, int o_f32, int64_t o_off, int64_t osh,
                                                       float* lse, int64_t lse_h, const float* gates,
                                                       int64_t gate_h) {
  MergeState<G, D> s1, s2;
  merge_run<G, D>(po, pml, 0, n_sel, ml_sh, s1);
  merge_run<G, D>(po, pml, n_sel, n_win, ml_sh, s2);
#pragma unroll
  for (int pp = 0; pp < MergeState<G, D>::PPT; ++pp) {
    const int i = threadIdx.x + 256 * pp;
    if (i >= MergeState<G, D>::NPOS) continue;
    const int h = i / (D / 2), d = 2 * (i - h * (D / 2));
    const float g0 = gates ? gates[(int64_t)h * gate_h] : 1.f, g1 = gates ? gates[(int64_t)h * gate_h + 1] : 1.f;
    const bool v1 = s1.L[pp] > 0.f, v2 = s2.L[pp] > 0.f;
    const float a0 = v1 ? s1.acc0[pp] / s1.L[pp] : 0.f, a1 = v1 ? s1.acc1[pp] / s1.L[pp] : 0.f;
    const float b0 = v2 ? s2.acc0[pp] / s2.L[pp] : 0.f, b1 = v2 ? s2.acc1[pp] / s2.L[pp] : 0.f;
    store_pair(o, o_f32, o_off + (int64_t)h * osh + d, g0 * a0 + g1 * b0, g0 * a1 + g1 * b1);
    if (d == 0) {
      lse[(int64_t)h * lse_h] = s1.L[pp] > 0.f ? (s1.M[pp] + log2f(s1.L[pp])) * kLn2 : -INFINITY;
      lse[(int64_t)h * lse_h + 1] = s2.L[pp] > 0.f ? (s2.M[pp] + log2f(s2.L[pp])) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace bsa
