// STQ1_0 encode and decode kernels for gfx950.
//
// Encoder (lemmy.durstig.online post 66506, "Scale and zero position are fit
// together"; alphasignal.ai summary bullets for the amax baseline): one
// wavefront per 256-weight block, one lane per group of four.  All encoder
// arithmetic is fp64 in a fixed order so the bytes match the reference
// encoder exactly:
//   - per group, the four lanes are added in lane order, a zeroed lane adding
//     +0.0;
//   - across the 64 groups, an xor butterfly over strides 1, 2, ..., 32, which
//     is the balanced tree of adjacent pairs (floating-point addition is
//     commutative, so every lane ends with the same bits);
//   - q*|w| of two fp32 values is exact in fp64, so contraction cannot change
//     it; the file is still built without contraction.
// d is stored as fp16 by fp64 -> fp32 -> fp16, round-to-nearest-even each
// time, clamped to 65504.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

// ---------------------------------------------------------------------------
// decode: one thread per group of four weights
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ q, int64_t n_groups, int n,
                                                         int nb, float* __restrict__ out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_groups) return;
  const int64_t blk = gid >> 6;  // row-major block index r*nb + b
  const int g = static_cast<int>(gid & 63);
  const int r = static_cast<int>(blk / nb);
  const int b = static_cast<int>(blk - static_cast<int64_t>(r) * nb);
  const uint8_t* p = q + block_offset(r, b, n, nb);
  const uint32_t d16 = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8);
  const uint32_t nib = (p[2 + 4 * (g >> 3) + (g & 3)] >> (4 * ((g >> 2) & 1))) & 15u;
  const uint32_t sel = (p[34 + 4 * (g >> 5) + (g & 3)] >> ((g >> 2) & 7)) & 1u;
  const uint32_t c = nib | (sel << 4);
  const uint32_t dbits = __float_as_uint(half_bits_to_float(d16));
  float* o = out + blk * kQK + 4 * g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = code_lane_value(c, j);
    o[j] = __uint_as_float(t == 0 ? 0u : (t < 0 ? (dbits ^ 0x80000000u) : dbits));
  }
}

// ---------------------------------------------------------------------------
// encode: one wavefront per block
// ---------------------------------------------------------------------------
// Cross-lane steps of the butterfly.  After the steps of stride < s every
// lane holds its aligned block of s lanes' result, so the partner block's
// value may come from any of its lanes: a quad permutation (strides 1, 2), a
// mirror inside 8 or 16 lanes (strides 4, 8; DPP moves, no LDS round trip),
// a swizzle inside 32 lanes (stride 16), and lanes 0 and 32 (stride 32).
// Each step adds (or ORs, or maxes) a lane's own block with its partner's, so
// every lane ends with the same bits as the xor butterfly.
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane l <- 7 - l within 8
constexpr int kDppMirror = 0x140;       // lane l <- 15 - l within 16
constexpr int kSwizzleXor16 = 0x401F;   // ds_swizzle bit mode: lane l <- l ^ 16 within 32

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}

// value of the partner block at butterfly stride s (1, 2, 4, 8 or 16)
template <int kStride>
__device__ __forceinline__ uint32_t partner_u32(uint32_t v) {
  if constexpr (kStride == 1) return dpp_u32<kDppQuadSwap1>(v);
  else if constexpr (kStride == 2) return dpp_u32<kDppQuadSwap2>(v);
  else if constexpr (kStride == 4) return dpp_u32<kDppHalfMirror>(v);
  else if constexpr (kStride == 8) return dpp_u32<kDppMirror>(v);
  else return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), kSwizzleXor16));
}

template <int kStride>
__device__ __forceinline__ double partner_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = partner_u32<kStride>(static_cast<uint32_t>(b));
  const uint64_t hi = partner_u32<kStride>(static_cast<uint32_t>(b >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// the halves' values at stride 32 (every lane of a half holds its half's value)
__device__ __forceinline__ double half_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), lane));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), lane));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// balanced tree of adjacent pairs over the 64 lanes (same bits in every lane)
__device__ __forceinline__ double wave_tree_sum(double v) {
  v = v + partner_f64<1>(v);
  v = v + partner_f64<2>(v);
  v = v + partner_f64<4>(v);
  v = v + partner_f64<8>(v);
  v = v + partner_f64<16>(v);
  return half_f64(v, 0) + half_f64(v, 32);
}

__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, partner_f64<1>(v));
  v = fmax(v, partner_f64<2>(v));
  v = fmax(v, partner_f64<4>(v));
  v = fmax(v, partner_f64<8>(v));
  v = fmax(v, partner_f64<16>(v));
  return fmax(half_f64(v, 0), half_f64(v, 32));
}

__device__ __forceinline__ double wls_scale(const double (&a)[4], const double (&q)[4], int z) {
  // weighted least squares scale for fixed zero lanes: sum(q|w|) / sum(q) over kept lanes
  double num = 0.0, den = 0.0;
  {
    const double n0 = (z == 0) ? 0.0 : q[0] * a[0];
    const double n1 = (z == 1) ? 0.0 : q[1] * a[1];
    const double n2 = (z == 2) ? 0.0 : q[2] * a[2];
    const double n3 = (z == 3) ? 0.0 : q[3] * a[3];
    num = ((n0 + n1) + n2) + n3;
    const double d0 = (z == 0) ? 0.0 : q[0];
    const double d1 = (z == 1) ? 0.0 : q[1];
    const double d2 = (z == 2) ? 0.0 : q[2];
    const double d3 = (z == 3) ? 0.0 : q[3];
    den = ((d0 + d1) + d2) + d3;
  }
  num = wave_tree_sum(num);
  den = wave_tree_sum(den);
  return den > 0.0 ? num / den : 0.0;
}

__device__ __forceinline__ int choose_zero(const double (&a)[4], const double (&q)[4], double d) {
  // zeroing lane j adds q_j * d * (2|w_j| - d) of weighted error; drop d >= 0
  int z = 0;
  double best = q[0] * (2.0 * a[0] - d);
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    const double c = q[j] * (2.0 * a[j] - d);
    if (c < best) {
      best = c;
      z = j;
    }
  }
  return z;
}

template <bool kWls>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, const float* __restrict__ imat,
                                                       int64_t n_blocks, int n, int nb, int64_t k, int rounds,
                                                       uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= n_blocks) return;  // uniform per wavefront
  const int64_t row = blk / nb;
  const int b = static_cast<int>(blk - row * nb);
  const int64_t col = static_cast<int64_t>(b) * kQK + 4 * lane;
  const float* wp = w + row * k + col;

  double a[4], q[4];
  bool neg[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = wp[j];
    a[j] = fabs(static_cast<double>(v));
    neg[j] = v < 0.0f;  // -0.0 counts as positive
    q[j] = imat ? static_cast<double>(imat[col + j]) : 1.0;
  }
  // starting pattern: zero the first smallest |w| of the group
  int z = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (a[j] < a[z]) z = j;

  double d;
  if (kWls) {
    for (int r = 0; r < rounds; ++r) {
      d = wls_scale(a, q, z);
      z = choose_zero(a, q, d);
    }
    d = wls_scale(a, q, z);
  } else {
    d = wave_max(fmax(fmax(a[0], a[1]), fmax(a[2], a[3])));
  }

  // fp16 scale: fp64 -> fp32 -> fp16, nearest-even each time, clamped to 65504
  float f = static_cast<float>(d);
  f = fminf(f, 65504.0f);
  const uint32_t d16 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));

  // code = 8*z + m, m's bit r set when the r-th kept lane is negative
  uint32_t m = 0;
  int r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j == z) continue;
    m |= static_cast<uint32_t>(neg[j]) << r;
    ++r;
  }
  const uint32_t c = 8u * static_cast<uint32_t>(z) + m;

  // pack: code words (8 groups each) and select words (32 groups each)
  const int g = lane;
  uint32_t qsw = (c & 15u) << (8 * (g & 3) + 4 * ((g >> 2) & 1));
  uint32_t qhw = (c >> 4) << (8 * (g & 3) + ((g >> 2) & 7));
  qsw |= partner_u32<1>(qsw);  // OR over the 8 lanes of a code word
  qsw |= partner_u32<2>(qsw);
  qsw |= partner_u32<4>(qsw);
  qhw |= partner_u32<1>(qhw);  // OR over the 32 lanes of a select word
  qhw |= partner_u32<2>(qhw);
  qhw |= partner_u32<4>(qhw);
  qhw |= partner_u32<8>(qhw);
  qhw |= partner_u32<16>(qhw);

  // 21 half-words per block: [d | 16 x code half-words | 4 x select half-words]
  const int i = lane;
  int src = 0;
  if (i >= 1 && i <= 16) src = 8 * ((i - 1) >> 1);
  else if (i >= 17 && i <= 20) src = 32 * ((i - 17) >> 1);
  const uint32_t vq = __shfl(qsw, src, 64);
  const uint32_t vh = __shfl(qhw, src, 64);
  uint32_t val;
  if (i == 0) val = d16;
  else if (i <= 16) val = (vq >> (16 * ((i - 1) & 1))) & 0xFFFFu;
  else val = (vh >> (16 * ((i - 17) & 1))) & 0xFFFFu;
  if (i < 21)
    reinterpret_cast<uint16_t*>(out + block_offset(static_cast<int>(row), b, n, nb))[i] = static_cast<uint16_t>(val);
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* q, int64_t n_rows, int64_t k, float* out, hipStream_t s) {
  const int64_t n_groups = n_rows * (k / 4);
  if (n_groups == 0) return hipSuccess;
  const int64_t grid = (n_groups + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, q, n_groups,
                     static_cast<int>(n_rows), static_cast<int>(k / kQK), out);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, const float* imatrix, int64_t n_rows, int64_t k, int encoder,
                           int rounds, uint8_t* out, hipStream_t s) {
  const int nb = static_cast<int>(k / kQK);
  const int64_t n_blocks = n_rows * nb;
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = (n_blocks + 3) / 4;
  if (encoder == 0)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, w, imatrix,
                       n_blocks, static_cast<int>(n_rows), nb, k, rounds, out);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, w, imatrix,
                       n_blocks, static_cast<int>(n_rows), nb, k, rounds, out);
  return hipGetLastError();
}

}  // namespace stq
