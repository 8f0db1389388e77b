// Split combine: merges the per-chunk softmax partials of each output row.
// With M = max_s m_s (log2 domain) and w_s = 2^(m_s - M):
//   out = sum_s w_s o_s / sum_s w_s l_s
// Empty chunks carry m = -inf, l = 0, o = 0 and drop out with w = 0.

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

__global__ __launch_bounds__(64) void k_combine(const float* __restrict__ part_o,
                                                const float* __restrict__ part_ml,
                                                float* __restrict__ out, int n_split, int D) {
  extern __shared__ float s_w[];   // n_split weights
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const float* ml = part_ml + (size_t)row * n_split * 2;

  float mx = -INFINITY;
  for (int s = lane; s < n_split; s += 64) mx = fmaxf(mx, ml[2 * s]);
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));

  float den = 0.0f;
  for (int s = lane; s < n_split; s += 64) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - mx);
    s_w[s] = w;
    den += w * ml[2 * s + 1];
  }
  for (int off = 1; off < 64; off <<= 1) den += shfl_xor_f(den, off);
  __syncthreads();

  const float inv = 1.0f / den;
  const float* o = part_o + (size_t)row * n_split * D;
  for (int d = lane; d < D; d += 64) {
    float num = 0.0f;
    for (int s = 0; s < n_split; ++s) num = fmaf(s_w[s], o[(size_t)s * D + d], num);
    out[(size_t)row * D + d] = num * inv;
  }
}

int launch_combine(const float* part_o, const float* part_ml, float* out, int n_rows, int n_split,
                   int head_dim, hipStream_t stream) {
  hipLaunchKernelGGL(k_combine, dim3(n_rows), dim3(64), n_split * sizeof(float), stream, part_o,
                     part_ml, out, n_split, head_dim);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
