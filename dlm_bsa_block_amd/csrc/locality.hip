// Locality pruning (active rows) as a launch of its own; the row job itself
// is in locality.h.
#include "internal.h"
#include "locality.h"

namespace bsa {

template <int DT>
__global__ __launch_bounds__(256) void active_rows_kernel(ActiveRowsArgs x) {
  __shared__ float sh[4];
  active_row_job<DT>(x, blockIdx.x, blockIdx.y, sh);
}

ActiveRowsArgs active_rows_args(const bsa_tensor& x, const bsa_tensor& y, float theta, uint8_t* mask, float* mse) {
  ActiveRowsArgs a;
  a.a = static_cast<const uint8_t*>(x.data);
  a.c = static_cast<const uint8_t*>(y.data);
  a.asb = x.stride_b; a.ash = x.stride_h; a.asl = x.stride_l;
  a.csb = y.stride_b; a.csh = y.stride_h; a.csl = y.stride_l;
  a.H = x.H; a.R = x.L; a.D = x.D; a.theta = theta; a.mask = mask; a.mse = mse;
  return a;
}

void launch_active_rows(const bsa_tensor& x, const bsa_tensor& y, float theta, uint8_t* mask, float* mse,
                        hipStream_t s) {
  const ActiveRowsArgs a = active_rows_args(x, y, theta, mask, mse);
  dim3 grid(x.L, x.B);
  if (x.dtype == BSA_BF16) hipLaunchKernelGGL(active_rows_kernel<BSA_BF16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(active_rows_kernel<BSA_F32>, grid, dim3(256), 0, s, a);
}

}  // namespace bsa
