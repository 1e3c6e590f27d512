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

// A pair's value at row offset i of a GEMV launched without its reduction:
// the split slots added in order from 0.0f (as the GEMV's own reduction adds
// them) for a valid pair with more than one slot, else the GEMV's direct
// output.  Four elements per thread in the SwiGLU pass: d_ff is a multiple of
// 256, so a float4 never straddles a row.
struct SplitRows {
  const float* y;
  const float* partial;
  int splits;
  const int32_t* pair_sub;
  const int32_t* pe;
  int n_experts;
  int64_t plane;  // n_pairs * row width
  __device__ __forceinline__ int slots(int p) const {
    if (!partial) return 1;
    const int e = pe[p];
    if (e < 0 || e >= n_experts) return 1;  // the GEMV wrote its NaN row directly
    return pair_sub ? splits * pair_sub[p] : splits;
  }
  // four values at element offset i (16-byte aligned); the loads of up to 16
  // slots are issued before their adds
  __device__ __forceinline__ float4 quad(int p, int64_t i) const {
    const int n_s = slots(p);
    if (n_s == 1) return *reinterpret_cast<const float4*>(y + i);
    constexpr int kBatch = 16;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < n_s; s0 += kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (s0 + j < n_s) v[j] = *reinterpret_cast<const float4*>(partial + (s0 + j) * plane + i);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (s0 + j < n_s) {
          acc.x += v[j].x;
          acc.y += v[j].y;
          acc.z += v[j].z;
          acc.w += v[j].w;
        }
      }
    }
    return acc;
  }
};

__global__ __launch_bounds__(256) void swiglu_kernel(SplitRows gu, int64_t quads, int64_t d_ff,
                                                     float* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= quads) return;
  const int64_t e = 4 * i;
  const int64_t p = e / d_ff;
  const int64_t c = e - p * d_ff;
  const float4 g = gu.quad(static_cast<int>(p), p * 2 * d_ff + c);
  const float4 u = gu.quad(static_cast<int>(p), p * 2 * d_ff + d_ff + c);
  float4 o;
  o.x = g.x / (1.0f + expf(-g.x)) * u.x;
  o.y = g.y / (1.0f + expf(-g.y)) * u.y;
  o.z = g.z / (1.0f + expf(-g.z)) * u.z;
  o.w = g.w / (1.0f + expf(-g.w)) * u.w;
  *reinterpret_cast<float4*>(h + e) = o;
}

// Workgroup (x, t): columns 256x.. of token t, so each routed pair's slot
// count is uniform.  Up to 8 pairs at a time: every load of their direct
// rows or split slots (at most kS slots a pair; kS = 0: any count, slot by
// slot) is issued before the adds, which keep the reduction's and the
// routing's order.
template <int kS>
__global__ __launch_bounds__(256) void combine_kernel(SplitRows z, const float* __restrict__ w, int top_k, int64_t n,
                                                      float* __restrict__ y) {
  const int64_t t = blockIdx.y;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n) return;
  constexpr int kK = 8;
  constexpr int kSlots = kS > 0 ? kS : 1;
  float acc = 0.0f;
  for (int k0 = 0; k0 < top_k; k0 += kK) {
    int ns[kK];
    float v[kK][kSlots];
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      const int64_t p = t * top_k + k0 + j;
      ns[j] = k0 + j < top_k ? z.slots(static_cast<int>(p)) : 0;
      if (ns[j] == 1) {
        v[j][0] = z.y[p * n + c];
      } else if (kS > 0) {
#pragma unroll
        for (int s = 0; s < kSlots; ++s)
          if (s < ns[j]) v[j][s] = z.partial[s * z.plane + p * n + c];
      }
    }
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      if (ns[j] == 0) continue;
      const int64_t p = t * top_k + k0 + j;
      float val;
      if (ns[j] == 1) {
        val = v[j][0];
      } else {
        val = 0.0f;
        if (kS > 0) {
#pragma unroll
          for (int s = 0; s < kSlots; ++s)
            if (s < ns[j]) val += v[j][s];
        } else {
          for (int s = 0; s < ns[j]; ++s) val += z.partial[s * z.plane + p * n + c];
        }
      }
      acc = fmaf(w[p], val, acc);
    }
  }
  y[t * n + c] = acc;
}

}  // namespace

hipError_t launch_swiglu(const float* gu, const GemvPartials& parts, const int32_t* pair_expert,
                               int64_t n_experts, int64_t n_pairs, int64_t d_ff, float* h, hipStream_t s) {
  const int64_t quads = n_pairs * d_ff / 4;
  if (quads == 0) return hipSuccess;
  const SplitRows r{gu, parts.partial, parts.splits, parts.pair_sub, pair_expert, static_cast<int>(n_experts),
                    n_pairs * 2 * d_ff};
  hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), 0, s, r,
                     quads, d_ff, h);
  return hipGetLastError();
}

hipError_t launch_combine(const float* z, const GemvPartials& parts, const int32_t* pair_expert, int64_t n_experts,
                          const float* w, int64_t n_tokens, int64_t top_k, int64_t n, float* y, hipStream_t s) {
  if (n_tokens == 0 || n == 0) return hipSuccess;
  const SplitRows r{z, parts.partial, parts.splits, parts.pair_sub, pair_expert, static_cast<int>(n_experts),
                    n_tokens * top_k * n};
  const int max_slots = parts.partial ? parts.max_slots : 1;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(n_tokens));
  const int k = static_cast<int>(top_k);
  if (max_slots <= 1) hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, s, r, w, k, n, y);
  else if (max_slots <= 2) hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, s, r, w, k, n, y);
  else if (max_slots <= 4) hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, s, r, w, k, n, y);
  else if (max_slots <= 8) hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, s, r, w, k, n, y);
  else hipLaunchKernelGGL(combine_kernel<0>, grid, dim3(256), 0, s, r, w, k, n, y);
  return hipGetLastError();
}



}  // namespace stq
