// Grouped STQ1_0 GEMM for the prefill path: for each expert e,
// Y[rows of e] = X[rows of e] * W_e^T, rows grouped by expert.
//
// The pages give the format and say STQ1_0 has GPU kernels (lemmy.durstig.online
// post 66506, "Runtime"); this is a dense contraction once the ternary
// patterns are expanded, so it runs on gfx950 matrix cores:
// v_mfma_f32_16x16x32_bf16, bf16 activations times exactly representable
// {-1, 0, +1} weights, fp32 accumulation.  The fp16 block scale d of each
// 256-weight block multiplies the block's partial product in fp32 (one FMA per
// output per block), so the products stay exact.
//
// Tiling: a workgroup (4 wavefronts) owns 128 output columns of one expert
// and up to 128 of its rows at a time; each wavefront owns 32 columns (two
// 16-column MFMA tiles) and every 16-row tile of the rows.  Per 256-weight
// block, the workgroup stages the activation tile (rows x 256 bf16) in LDS;
// each lane expands its own weights straight from the packed block: in MFMA
// step s (32 k values) lane quarter j takes groups 8s+j and 8s+4+j, i.e. the
// two nibbles of byte j of code word s, and the activation fragment is read
// with the same k order, so A and B agree on every k.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCols = 128;    // output columns per workgroup
constexpr int kMRows = 128;   // rows per pass
constexpr int kMSub = kMRows / 16;
constexpr int kPitch = 264;   // LDS row pitch of the activation tile, bf16 elements

struct GArgs {
  const uint8_t* w;
  int64_t estride;
  int n;
  int nb;
  const uint16_t* x;
  int64_t k;
  const int32_t* offsets;
  int total_m;
  float* y;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__global__ __launch_bounds__(256) void grouped_gemm_kernel(GArgs a) {
  __shared__ uint16_t s_x[kMRows * kPitch];
  __shared__ uint2 s_lut[32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.y;
  const int n0 = blockIdx.x * kCols;
  // rows of expert e, clamped to [0, total_m] so bad offsets cannot reach outside x or y
  const int row0 = max(0, min(a.offsets[e], a.total_m));
  const int row1 = max(row0, min(a.offsets[e + 1], a.total_m));
  if (row1 <= row0) return;

  // pattern table: code -> four bf16 of {-1, 0, +1}
  if (tid < 32) {
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = code_lane_value(static_cast<uint32_t>(tid), j);
      h[j] = t == 0 ? 0u : (t > 0 ? 0x3F80u : 0xBF80u);
    }
    s_lut[tid] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }

  const int col_in = lane & 15;   // column inside a 16-wide tile (B and D)
  const int quarter = lane >> 4;  // k quarter (A, B) / row quarter (D)
  int ncol[2];
  const uint8_t* wrow[2];   // block 0 of this lane's weight row; block b is b * tile_rows * 42 further
  int64_t bstep[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ncol[t] = n0 + 32 * wave + 16 * t + col_in;
    const int nc = ncol[t] < a.n ? ncol[t] : a.n - 1;
    wrow[t] = a.w + static_cast<int64_t>(e) * a.estride + block_offset(nc, 0, a.n, a.nb);
    bstep[t] = static_cast<int64_t>(min(kTileRows, a.n - (nc & ~(kTileRows - 1)))) * kBlockBytes;
  }

  for (int m0 = row0; m0 < row1; m0 += kMRows) {
    const int mrows = min(kMRows, row1 - m0);
    const int nms = (mrows + 15) >> 4;
    f32x4_t acc[kMSub][2];
#pragma unroll
    for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[ms][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Block nxt[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) nxt[t] = load_block_global(wrow[t]);

    for (int b = 0; b < a.nb; ++b) {
      Block blk[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        blk[t] = nxt[t];
        if (b + 1 < a.nb) nxt[t] = load_block_global(wrow[t] + static_cast<int64_t>(b + 1) * bstep[t]);
      }
      __syncthreads();  // previous block's reads of s_x are done
      // stage activations rows [m0, m0+128) x k [256b, 256b+256) as bf16, zero past the expert
#pragma unroll
      for (int u = 0; u < (kMRows * 32) / 256; ++u) {
        const int c = tid + 256 * u;
        const int r = c >> 5, c16 = c & 31;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < mrows)
          v = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(m0 + r) * a.k + 256 * b + 8 * c16);
        *reinterpret_cast<uint4*>(&s_x[r * kPitch + 8 * c16]) = v;
      }
      __syncthreads();

      f32x4_t part[kMSub][2];
#pragma unroll
      for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
        for (int t = 0; t < 2; ++t) part[ms][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8_t bfrag[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t Q = blk[t].qs[s];
          const uint32_t H = blk[t].qh[s >> 2] >> (8 * quarter + 2 * (s & 3));
          const uint32_t c1 = ((Q >> (8 * quarter)) & 15u) | ((H & 1u) << 4);
          const uint32_t c2 = ((Q >> (8 * quarter + 4)) & 15u) | ((H & 2u) << 3);
          const uint2 p1 = s_lut[c1];
          const uint2 p2 = s_lut[c2];
          bfrag[t] = as_bf16x8(u32x4_t{p1.x, p1.y, p2.x, p2.y});
        }
#pragma unroll
        for (int ms = 0; ms < kMSub; ++ms) {
          if (ms < nms) {
            const uint16_t* ap = &s_x[(16 * ms + col_in) * kPitch + 32 * s + 4 * quarter];
            const uint2 a1 = *reinterpret_cast<const uint2*>(ap);
            const uint2 a2 = *reinterpret_cast<const uint2*>(ap + 16);
            const bf16x8_t afrag = as_bf16x8(u32x4_t{a1.x, a1.y, a2.x, a2.y});
#pragma unroll
            for (int t = 0; t < 2; ++t)
              part[ms][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[t], part[ms][t], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float d = half_bits_to_float(blk[t].d16);
#pragma unroll
        for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ms][t][r] = fmaf(d, part[ms][t][r], acc[ms][t][r]);
      }
    }

    // D layout: lane holds rows 4*quarter + r of the 16-row tile, column col_in
#pragma unroll
    for (int ms = 0; ms < kMSub; ++ms) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (ncol[t] >= a.n) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 16 * ms + 4 * quarter + r;
          if (rr < mrows) a.y[static_cast<int64_t>(m0 + rr) * a.n + ncol[t]] = acc[ms][t][r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& ga, hipStream_t s) {
  if (ga.total_m == 0 || ga.n == 0 || ga.n_experts == 0) return hipSuccess;
  GArgs a{};
  a.w = ga.w_table;
  a.estride = ga.expert_stride;
  a.n = static_cast<int>(ga.n);
  a.nb = static_cast<int>(ga.k / kQK);
  a.x = ga.x;
  a.k = ga.k;
  a.offsets = ga.offsets;
  a.total_m = static_cast<int>(ga.total_m);
  a.y = ga.y;
  const dim3 grid(static_cast<unsigned>((ga.n + kCols - 1) / kCols), static_cast<unsigned>(ga.n_experts));
  hipLaunchKernelGGL(grouped_gemm_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace stq
