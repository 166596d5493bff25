// Block summaries: one coalesced pass over K (or Q) producing the per-block
// mean and the per-band mean energy (Prism, technical summary sec. 1-2).
//
// One workgroup per (block, head, batch).  A row of D elements is read by
// D/8 lanes with 16-byte (bf16) or 32-byte (f32) loads, so each wave streams
// whole contiguous rows; up to four passes of loads are in flight per thread.
// Reductions run in a fixed order, so results are bitwise repeatable.
#include "common.h"
#include "internal.h"

namespace bsa {

template <int DT, int D>
__global__ __launch_bounds__(256) void summaries_kernel(const uint8_t* __restrict__ base, int64_t sb, int64_t sh,
                                                        int64_t sl, int L, int NB, int BS, int first, int layout,
                                                        float* __restrict__ mean, float* __restrict__ energy) {
  constexpr int LPR = D / 8;        // lanes per row
  constexpr int RPP = 256 / LPR;    // rows per pass
  constexpr int ES = DT == BSA_BF16 ? 2 : 4;
  constexpr int CH = 4;             // passes whose loads are issued together
  __shared__ float red[RPP][D + 4];
  __shared__ float ered[4][2];

  const int j = first + blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z, H = gridDim.y;
  const int tid = threadIdx.x, c = tid % LPR, rg = tid / LPR;
  const int t0 = j * BS;
  const int n = min(BS, L - t0);
  const uint8_t* p = base + ((int64_t)b * sb + (int64_t)h * sh + (int64_t)t0 * sl) * ES + c * 8 * ES;
  const int band = band_of_dim(c * 8, D, layout);   // 8 consecutive dims never straddle a band edge

  float sum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum[i] = 0.f;
  float e = 0.f;
  for (int r0 = 0; r0 < n; r0 += CH * RPP) {
    // rows past the block's end load its last row and are zeroed: a load under a branch
    // would make the compiler wait for each pass before requesting the next
    float v[CH][8];
#pragma unroll
    for (int k = 0; k < CH; ++k) load8<DT>(p + (int64_t)min(r0 + k * RPP + rg, n - 1) * sl * ES, v[k]);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const bool in = r0 + k * RPP + rg < n;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[k][i] = in ? v[k][i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) { sum[i] += v[k][i]; e = fmaf(v[k][i], v[k][i], e); }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rg][c * 8 + i] = sum[i];
  float ef = band == 0 ? e : 0.f, es = band == 0 ? 0.f : e;
  ef = wave_sum(ef);
  es = wave_sum(es);
  if ((tid & 63) == 0) { ered[tid >> 6][0] = ef; ered[tid >> 6][1] = es; }
  __syncthreads();
  const float inv = 1.0f / (float)n;
  const int64_t row = ((int64_t)b * H + h) * NB + j;
  for (int d = tid; d < D; d += 256) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < RPP; ++g) t += red[g][d];
    mean[row * D + d] = t * inv;
  }
  if (energy != nullptr && tid < 2) {
    float t = ered[0][tid] + ered[1][tid] + ered[2][tid] + ered[3][tid];
    energy[row * 2 + tid] = t * inv;
  }
}

void launch_summaries(const bsa_tensor& x, int block, int layout, int first, int nblk, float* mean, float* energy,
                      hipStream_t s) {
  const int NB = (int)ceil_div(x.L, block);
  dim3 grid(nblk, x.H, x.B);
  const uint8_t* base = static_cast<const uint8_t*>(x.data);
#define BSA_SUM(DT, DD)                                                                                  \
  hipLaunchKernelGGL((summaries_kernel<DT, DD>), grid, dim3(256), 0, s, base, x.stride_b, x.stride_h,   \
                     x.stride_l, x.L, NB, block, first, layout, mean, energy)
  if (x.dtype == BSA_BF16) {
    if (x.D == 128) BSA_SUM(BSA_BF16, 128); else BSA_SUM(BSA_BF16, 64);
  } else {
    if (x.D == 128) BSA_SUM(BSA_F32, 128); else BSA_SUM(BSA_F32, 64);
  }
#undef BSA_SUM
}

}  // namespace bsa
