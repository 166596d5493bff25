// Locality pruning for a block-wise diffusion LM denoising step (LoSA page,
// technical summary sec. 2): a query row is active when the mean squared
// change of its query vectors since the previous step, over all heads and
// dims, exceeds a threshold; stable rows keep their cached output.
//
// One workgroup per (row, batch).  Each thread accumulates a fixed strided
// subset in fp32, then a fixed-order tree reduction, so the decision is
// repeatable bit for bit.
#include "common.h"
#include "internal.h"

namespace bsa {

template <int DT>
__global__ __launch_bounds__(256) void active_rows_kernel(const uint8_t* __restrict__ a, int64_t asb, int64_t ash,
                                                          int64_t asl, const uint8_t* __restrict__ c, int64_t csb,
                                                          int64_t csh, int64_t csl, int H, int R, int D,
                                                          float theta, uint8_t* __restrict__ mask,
                                                          float* __restrict__ mse) {
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  __shared__ float sh[4];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int per_head = D / 8;
  float acc = 0.f;
  for (int i = tid; i < H * per_head; i += 256) {
    const int h = i / per_head, d8 = (i - h * per_head) * 8;
    float x[8], y[8];
    load8<DT>(a + ((int64_t)b * asb + (int64_t)h * ash + (int64_t)r * asl + d8) * ES, x);
    load8<DT>(c + ((int64_t)b * csb + (int64_t)h * csh + (int64_t)r * csl + d8) * ES, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = x[e] - y[e];
      acc = fmaf(d, d, acc);
    }
  }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) sh[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float m = (sh[0] + sh[1] + sh[2] + sh[3]) / (float)((int64_t)H * D);
    mask[(int64_t)b * R + r] = m > theta ? 1 : 0;
    if (mse) mse[(int64_t)b * R + r] = m;
  }
}

void launch_active_rows(const bsa_tensor& x, const bsa_tensor& y, float theta, uint8_t* mask, float* mse,
                        hipStream_t s) {
  dim3 grid(x.L, x.B);
  const uint8_t* a = static_cast<const uint8_t*>(x.data);
  const uint8_t* c = static_cast<const uint8_t*>(y.data);
  if (x.dtype == BSA_BF16)
    hipLaunchKernelGGL(active_rows_kernel<BSA_BF16>, grid, dim3(256), 0, s, a, x.stride_b, x.stride_h, x.stride_l, c,
                       y.stride_b, y.stride_h, y.stride_l, x.H, x.L, x.D, theta, mask, mse);
  else
    hipLaunchKernelGGL(active_rows_kernel<BSA_F32>, grid, dim3(256), 0, s, a, x.stride_b, x.stride_h, x.stride_l, c,
                       y.stride_b, y.stride_h, y.stride_l, x.H, x.L, x.D, theta, mask, mse);
}

}  // namespace bsa
