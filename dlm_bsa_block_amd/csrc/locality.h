// Locality pruning for a block-wise diffusion LM denoising step (LoSA page,
// technical summary sec. 2): a query row is active when the mean squared
// change of its query vectors since the previous step, over all heads and
// dims, exceeds a threshold; stable rows keep their cached output.
//
// One 256-thread workgroup per (row, batch).  Each thread accumulates a fixed
// strided subset in fp32, then a fixed-order tree reduction, so the decision
// is repeatable bit for bit -- also where the denoising step runs it inside
// its logits launch.
#pragma once
#include "common.h"
#include "internal.h"

namespace bsa {

template <int DT>
__device__ __forceinline__ void active_row_job(const ActiveRowsArgs& x, int r, int b, float* sh4) {
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  const int tid = threadIdx.x;
  const int per_head = x.D / 8;
  float acc = 0.f;
  for (int i = tid; i < x.H * per_head; i += 256) {
    const int h = i / per_head, d8 = (i - h * per_head) * 8;
    float p[8], q[8];
    load8<DT>(x.a + ((int64_t)b * x.asb + (int64_t)h * x.ash + (int64_t)r * x.asl + d8) * ES, p);
    load8<DT>(x.c + ((int64_t)b * x.csb + (int64_t)h * x.csh + (int64_t)r * x.csl + d8) * ES, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = p[e] - q[e];
      acc = fmaf(d, d, acc);
    }
  }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) sh4[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float m = (sh4[0] + sh4[1] + sh4[2] + sh4[3]) / (float)((int64_t)x.H * x.D);
    x.mask[(int64_t)b * x.R + r] = m > x.theta ? 1 : 0;
    if (x.mse) x.mse[(int64_t)b * x.R + r] = m;
  }
}

}  // namespace bsa
