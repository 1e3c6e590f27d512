// Elementwise parts of a MoE layer's routed-expert FFN for decode.
//
// SwiGLU activation: each pair's gate/up row [gate (d_ff) | up (d_ff)] gives
// h = silu(gate) * up with silu(v) = v / (1 + exp(-v)), in fp32, once per
// element, ahead of the down projection (which then reads plain fp32 rows).
//
// Routing-weighted combine of the expert outputs: each token's output is the
// sum, in routing order, of its experts' outputs scaled by the routing
// weights (top-k of the routed experts, traictory.com "Tencent's 200GB
// Hy4-preview ...", "The claim, stated precisely").  One thread per output
// element; fixed order, so repeated calls give identical bits.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

// Four elements per thread: d_ff is a multiple of 256, so a float4 never
// straddles a row.
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ gu, int64_t quads, int64_t d_ff,
                                                     float* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= quads) return;
  const int64_t e = 4 * i;
  const int64_t p = e / d_ff;
  const int64_t c = e - p * d_ff;
  const float4 g = *reinterpret_cast<const float4*>(gu + p * 2 * d_ff + c);
  const float4 u = *reinterpret_cast<const float4*>(gu + p * 2 * d_ff + d_ff + c);
  float4 o;
  o.x = g.x / (1.0f + expf(-g.x)) * u.x;
  o.y = g.y / (1.0f + expf(-g.y)) * u.y;
  o.z = g.z / (1.0f + expf(-g.z)) * u.z;
  o.w = g.w / (1.0f + expf(-g.w)) * u.w;
  *reinterpret_cast<float4*>(h + e) = o;
}

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

hipError_t launch_swiglu(const float* gu, int64_t n_pairs, int64_t d_ff, float* h, hipStream_t s) {
  const int64_t quads = n_pairs * d_ff / 4;
  if (quads == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), 0, s, gu, quads,
                     d_ff, h);
  return hipGetLastError();
}

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
