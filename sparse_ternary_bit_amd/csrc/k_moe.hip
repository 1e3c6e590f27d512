// Routing-weighted combine of a MoE layer's expert outputs for decode: each
// token's output is the sum, in routing order, of its experts' outputs
// scaled by the routing weights (top-k of the routed experts,
// traictory.com "Tencent's 200GB Hy4-preview ...", "The claim, stated
// precisely").  One thread per output element; fixed order, so repeated
// calls give identical bits.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ z, const float* __restrict__ w,
                                                      int64_t total, int top_k, int64_t n, float* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t t = i / n;
  const int64_t c = i - t * n;
  float acc = 0.0f;
  for (int k = 0; k < top_k; ++k) {
    const int64_t p = t * top_k + k;
    acc = fmaf(w[p], z[p * n + c], acc);
  }
  y[i] = acc;
}

}  // namespace

hipError_t launch_combine(const float* z, const float* w, int64_t n_tokens, int64_t top_k, int64_t n, float* y,
                          hipStream_t s) {
  const int64_t total = n_tokens * n;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, z, w, total,
                     static_cast<int>(top_k), n, y);
  return hipGetLastError();
}

}  // namespace stq
