// Measurement references (not part of the method).
//
// Streaming-read reference for the HBM roofline: reads a device buffer once
// with 16-byte loads (four in flight per thread, grid-stride) and folds every
// word of every load into one value (so no load can be narrowed), so the rate
// it reaches is what this GPU sustains for plain reads, measured beside the
// decode GEMV's effective bandwidth.
#include "stq_launch.hpp"

namespace stq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeGrid = 8192;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t s = 0;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  auto fold = [](u32x4_t v) { return (v.x ^ v.y) + (v.z ^ v.w); };
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    s += (fold(a) ^ fold(b)) + (fold(c) ^ fold(d));
  }
  for (; i < n; i += stride) s += fold(p[i]);
  // the fold is kept only if it can reach memory; the one-word sink is
  // written by at most the threads whose fold matches a fixed tag
  if (s == 0x5EED5EEDu) sink[0] = s;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < kProbeGrid ? want : kProbeGrid);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, s, static_cast<const u32x4_t*>(buf), n, sink);
  return hipGetLastError();
}

}  // namespace stq

// Matrix-core reference for the grouped GEMM's MFMA roofline: every
// wavefront runs `iters` rounds of eight independent
// v_mfma_f32_16x16x32_bf16 (no memory traffic, no other work), so the rate
// is what the matrix cores sustain for this instruction on this GPU.
namespace stq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* __restrict__ sink) {
  // operands from the lane index, bf16 1.0 and 2^-8 steps: finite, nonzero
  const uint32_t lane = threadIdx.x & 63;
  const u32x4_t ua = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4_t ub = {0x3B803B80u + lane, 0x3B803B80u, 0x3B803B80u, 0x3B803B80u + (lane << 16)};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ua);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, ub);
  f32x4_t c[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
  if (s == -1.0f) sink[0] = s;  // never true (all sums are positive); keeps the loop
}

// LDS read reference: every wavefront reads a 32 KB LDS buffer in a loop,
// eight reads in flight per round, with one of two access forms:
//   mode 0: 16-byte reads, a wavefront's 64 lanes one contiguous 1 KB run
//           (conflict free), the form of the grouped GEMM's activation reads;
//   mode 1: two 4-byte reads 128 bytes apart at a per-lane code (0..31) of a
//           32-entry table (one ds_read2_b32), the form of its pattern reads.
// Each read is folded into an accumulator (one or two XORs), so the loop is
// bound by the LDS, not by the VALU.
__global__ __launch_bounds__(256) void lds_read_kernel(int mode, int64_t iters, uint32_t* __restrict__ sink) {
  __shared__ u32x4_t buf[kLdsProbeWords];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsProbeWords; i += 256) buf[i] = u32x4_t{uint32_t(i), uint32_t(i) * 3u, ~uint32_t(i), uint32_t(i) ^ 0x55u};
  __syncthreads();
  uint32_t acc[kLdsReads];
#pragma unroll
  for (int j = 0; j < kLdsReads; ++j) acc[j] = 0;
  if (mode == 0) {
    // read j of a round: wavefront-contiguous 1 KB run number (wave * 8 + j) mod 32
    const u32x4_t* p[kLdsReads];
#pragma unroll
    for (int j = 0; j < kLdsReads; ++j) p[j] = buf + (((wave * kLdsReads + j) & 31) * 64 + lane);
    for (int64_t i = 0; i < iters; ++i) {
      asm volatile("" ::: "memory");  // the buffer may have changed: read it again
#pragma unroll
      for (int j = 0; j < kLdsReads; ++j) {
        const u32x4_t v = *p[j];
        acc[j] ^= (v.x ^ v.y) ^ (v.z ^ v.w);
      }
    }
  } else {
    // codes of a fixed per-lane pseudo-random sequence (a 32-bit LCG), one per read
    const uint32_t* t = reinterpret_cast<const uint32_t*>(buf);
    uint32_t code[kLdsReads];
    uint32_t x = 0x9E3779B9u * static_cast<uint32_t>(lane + 1) + static_cast<uint32_t>(wave);
#pragma unroll
    for (int j = 0; j < kLdsReads; ++j) {
      x = x * 1664525u + 1013904223u;
      code[j] = x >> 27;
    }
    for (int64_t i = 0; i < iters; ++i) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < kLdsReads; ++j) acc[j] ^= t[code[j]] ^ t[code[j] + 32];
    }
  }
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < kLdsReads; ++j) s += acc[j];
  if (s == 0x5EED5EEDu) sink[0] = s;
}

}  // namespace

hipError_t launch_mfma_loop(int64_t iters, float* sink, hipStream_t s) {
  if (iters <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(kMfmaProbeGrid), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_lds_read(int mode, int64_t iters, uint32_t* sink, hipStream_t s) {
  if (iters <= 0) return hipSuccess;
  hipLaunchKernelGGL(lds_read_kernel, dim3(kLdsProbeGrid), dim3(256), 0, s, mode, iters, sink);
  return hipGetLastError();
}

}  // namespace stq
