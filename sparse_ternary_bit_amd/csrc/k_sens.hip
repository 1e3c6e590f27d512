// Layer-sensitivity kernels for gfx950: reconstruction error of a quantized
// matrix under calibration activations, scored with the full Hessian
// H = X^T X and with its diagonal alone, and the plain 2-bit format used as
// the larger partner when layers are allocated by error reduction per byte
// (lemmy.durstig.online post 66506, paragraph "Full-Hessian scoring";
// alphasignal.ai summary, bullet "Full-Hessian scoring").
//
// With D = W - W_hat (fp64, [n, k]) and calibration rows x_i (fp32, [N, k]):
//   full[r] = sum_i (D_r . x_i)^2 = D_r H D_r^T
//   diag[r] = sum_k H_kk D_rk^2,      H_kk = sum_i x_ik^2
// full is a dense contraction, P = D X^T, done on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64): fp32 operands are exact in fp64, so the only
// rounding is the fp64 accumulation.  diag rides along with the staging of
// D in the workgroups of the first calibration tile.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

typedef double double4_t __attribute__((ext_vector_type(4)));

constexpr int kSensRows = 64;   // weight rows per workgroup
constexpr int kSensCal = 64;    // calibration rows per workgroup
constexpr int kSensK = 32;      // k per LDS chunk
constexpr int kDPitch = kSensK + 2;   // doubles per staged D row (272 B: conflict-free b128 reads)
constexpr int kXPitch = kSensK + 4;   // floats per staged x row (144 B)

// ---------------------------------------------------------------------------
// H_kk = sum over calibration rows of x_ik^2 (fp64).  A workgroup owns 32
// columns; its 8 row slices (slice s takes rows s, s+8, s+16, ...) add their
// rows in order, then the 8 slice sums are added in slice order: a fixed
// order, independent of scheduling.
// ---------------------------------------------------------------------------
constexpr int kHdCols = 32;
constexpr int kHdSlices = 8;

__global__ __launch_bounds__(256) void hdiag_kernel(const float* __restrict__ x, int64_t n_cal, int64_t k,
                                                    double* __restrict__ hd) {
  __shared__ double part[kHdSlices][kHdCols];
  const int tx = threadIdx.x & (kHdCols - 1), ty = threadIdx.x / kHdCols;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kHdCols + tx;
  double s = 0.0;
  if (c < k) {
    int64_t i = ty;
    for (; i + 3 * kHdSlices < n_cal; i += 4 * kHdSlices) {
      const double v0 = static_cast<double>(x[i * k + c]);
      const double v1 = static_cast<double>(x[(i + kHdSlices) * k + c]);
      const double v2 = static_cast<double>(x[(i + 2 * kHdSlices) * k + c]);
      const double v3 = static_cast<double>(x[(i + 3 * kHdSlices) * k + c]);
      s += v0 * v0;
      s += v1 * v1;
      s += v2 * v2;
      s += v3 * v3;
    }
    for (; i < n_cal; i += kHdSlices) {
      const double v = static_cast<double>(x[i * k + c]);
      s += v * v;
    }
  }
  part[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && c < k) {
    double t = part[0][tx];
#pragma unroll
    for (int j = 1; j < kHdSlices; ++j) t += part[j][tx];
    hd[c] = t;
  }
}

// One staged float4 slot: D = w - w_hat in fp64 (zero for rows past the
// end), x as fp32 (zero past the end), and, for the diagonal score, the
// running sum of H_kk D_k^2 over the slot's four columns in column order.
__device__ __forceinline__ void stage_store(double* dp, float* xp, float4 wv, float4 hv, float4 xv, bool wok,
                                            bool xok, bool with_diag, const double* h, double& dacc) {
  const double d0 = wok ? static_cast<double>(wv.x) - static_cast<double>(hv.x) : 0.0;
  const double d1 = wok ? static_cast<double>(wv.y) - static_cast<double>(hv.y) : 0.0;
  const double d2 = wok ? static_cast<double>(wv.z) - static_cast<double>(hv.z) : 0.0;
  const double d3 = wok ? static_cast<double>(wv.w) - static_cast<double>(hv.w) : 0.0;
  dp[0] = d0;
  dp[1] = d1;
  dp[2] = d2;
  dp[3] = d3;
  *reinterpret_cast<float4*>(xp) = xok ? xv : make_float4(0.f, 0.f, 0.f, 0.f);
  if (with_diag) {
    dacc += h[0] * (d0 * d0);
    dacc += h[1] * (d1 * d1);
    dacc += h[2] * (d2 * d2);
    dacc += h[3] * (d3 * d3);
  }
}

// one chunk's global loads of one thread: two float4 slots of w, w_hat and x
struct Stage {
  float4 w0, w1, h0, h1, x0, x1;
};

struct SensSmem {
  double d[2][kSensRows][kDPitch];
  float x[2][kSensCal][kXPitch];
};

// One workgroup: 64 weight rows x 64 calibration rows, 4 waves as 2 x 2, a
// wave owning 32 x 32 of P as 2 x 2 tiles of 16 x 16.  Per 32-wide k chunk a
// lane (i = lane & 15, g = lane >> 4) feeds k = 8g + s to MFMA step s, so its
// 8 operands of a tile row are one contiguous 64-byte run in LDS.
__global__ __launch_bounds__(256) void layer_errors_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ w_hat, int n_rows, int64_t k,
                                                           const float* __restrict__ x, int n_cal,
                                                           const double* __restrict__ hd,
                                                           double* __restrict__ partial,
                                                           double* __restrict__ err_diag, int ctiles) {
  __shared__ SensSmem sm;
  // workgroup -> (row tile, calibration tile): ids are dealt to the 8 XCDs
  // round robin, so id = 8 * (ctiles * g + ct) + x holds row tile 8g + x
  // with every calibration tile on XCD x, dispatched together; they stream
  // the same weight rows through that XCD's L2
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int ct = local % ctiles;
  const int rt = (local / ctiles) * 8 + xcd;
  const int r0 = rt * kSensRows;
  if (r0 >= n_rows) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int c0 = ct * kSensCal;
  const bool with_diag = ct == 0;
  const int n_chunks = static_cast<int>(k / kSensK);

  // staging: thread t moves float4 slots t and t + 256 of each 64 x 32 tile
  // (slot -> row slot >> 3, columns 4 * (slot & 7) .. + 3).  Rows past the
  // end load the last valid row and are zeroed after the load.
  const int c4 = tid & 7;
  const int srow0 = tid >> 3, srow1 = srow0 + 32;
  const bool wok0 = r0 + srow0 < n_rows, wok1 = r0 + srow1 < n_rows;
  const bool xok0 = c0 + srow0 < n_cal, xok1 = c0 + srow1 < n_cal;
  const float* wp0 = w + static_cast<int64_t>(min(r0 + srow0, n_rows - 1)) * k + 4 * c4;
  const float* wp1 = w + static_cast<int64_t>(min(r0 + srow1, n_rows - 1)) * k + 4 * c4;
  const float* hp0 = w_hat + static_cast<int64_t>(min(r0 + srow0, n_rows - 1)) * k + 4 * c4;
  const float* hp1 = w_hat + static_cast<int64_t>(min(r0 + srow1, n_rows - 1)) * k + 4 * c4;
  const float* xp0 = x + static_cast<int64_t>(min(c0 + srow0, n_cal - 1)) * k + 4 * c4;
  const float* xp1 = x + static_cast<int64_t>(min(c0 + srow1, n_cal - 1)) * k + 4 * c4;
  double dacc0 = 0.0, dacc1 = 0.0;

  // Global loads run two chunks ahead (two register sets, used alternately),
  // so a chunk's weights have two chunks' MFMA time to arrive.
  auto load = [&](Stage& st, int ch) {
    const int64_t kc = static_cast<int64_t>(ch) * kSensK;
    st.w0 = *reinterpret_cast<const float4*>(wp0 + kc);
    st.w1 = *reinterpret_cast<const float4*>(wp1 + kc);
    st.h0 = *reinterpret_cast<const float4*>(hp0 + kc);
    st.h1 = *reinterpret_cast<const float4*>(hp1 + kc);
    st.x0 = *reinterpret_cast<const float4*>(xp0 + kc);
    st.x1 = *reinterpret_cast<const float4*>(xp1 + kc);
  };
  auto store = [&](const Stage& st, int ch, int buf) {
    const double* h = hd + static_cast<int64_t>(ch) * kSensK + 4 * c4;
    stage_store(sm.d[buf][srow0] + 4 * c4, sm.x[buf][srow0] + 4 * c4, st.w0, st.h0, st.x0, wok0, xok0, with_diag, h,
                dacc0);
    stage_store(sm.d[buf][srow1] + 4 * c4, sm.x[buf][srow1] + 4 * c4, st.w1, st.h1, st.x1, wok1, xok1, with_diag, h,
                dacc1);
  };

  double4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = double4_t{0.0, 0.0, 0.0, 0.0};

  const int li = lane & 15, lg = lane >> 4;
  auto compute = [&](int buf) {
    double av[2][8];
    float bv[2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const double* p = &sm.d[buf][32 * wr + 16 * a + li][8 * lg];
#pragma unroll
      for (int s = 0; s < 8; ++s) av[a][s] = p[s];
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float* p = &sm.x[buf][32 * wc + 16 * b + li][8 * lg];
#pragma unroll
      for (int s = 0; s < 8; ++s) bv[b][s] = p[s];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const double b0 = static_cast<double>(bv[0][s]);
      const double b1 = static_cast<double>(bv[1][s]);
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[0][s], b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[0][s], b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[1][s], b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[1][s], b1, acc[1][1], 0, 0, 0);
    }
  };

  Stage sa, sb;
  load(sa, 0);
  if (n_chunks > 1) load(sb, 1);
  store(sa, 0, 0);
  __syncthreads();
  // chunk ch computes from LDS buffer ch & 1; set A holds even chunks, set B odd ones
  for (int ch = 0; ch < n_chunks; ch += 2) {
    if (ch + 2 < n_chunks) load(sa, ch + 2);
    compute(0);
    if (ch + 1 < n_chunks) store(sb, ch + 1, 1);  // buffer 1 was last read before the previous barrier
    __syncthreads();
    if (ch + 1 >= n_chunks) break;
    if (ch + 3 < n_chunks) load(sb, ch + 3);
    compute(1);
    if (ch + 2 < n_chunks) store(sa, ch + 2, 0);
    __syncthreads();
  }

  // P tile (a, b): the fp64 16x16x4 result keeps row 4 * j + lg of the tile
  // in element j (j = 0..3) of lane 16 * lg + li, column li.  Sum the
  // squares over this wave's 32 calibration columns: the two tiles b in order,
  // then the 16 lanes of a row group by an xor butterfly.
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      double s = acc[a][0][j] * acc[a][0][j];
      s += acc[a][1][j] * acc[a][1][j];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) s += __shfl_xor(s, m, 64);
      const int gr = r0 + 32 * wr + 16 * a + 4 * j + lg;
      if (li == 0 && gr < n_rows)
        partial[(static_cast<int64_t>(ct) * 2 + wc) * n_rows + gr] = s;
    }
  }
  if (with_diag) {
    double s0 = dacc0, s1 = dacc1;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      s0 += __shfl_xor(s0, m, 64);
      s1 += __shfl_xor(s1, m, 64);
    }
    if (c4 == 0 && wok0) err_diag[r0 + srow0] = s0;
    if (c4 == 0 && wok1) err_diag[r0 + srow1] = s1;
  }
}

// full[r] = sum over partial slots, in slot order
__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partial, int n_slots,
                                                           int n_rows, double* __restrict__ full) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n_rows) return;
  double s = 0.0;
  for (int p = 0; p < n_slots; ++p) s += partial[static_cast<int64_t>(p) * n_rows + r];
  full[r] = s;
}

// ---------------------------------------------------------------------------
// 2-bit stand-in format: per 256 weights s = fp16(rms / 2), levels +-s, +-3s
// ---------------------------------------------------------------------------
// One wavefront per block, one lane per group of four.  The sum of squares is
// fp64 (squares of fp32 values are exact), the four lanes of a group in lane
// order, then the xor butterfly over the 64 groups.
__global__ __launch_bounds__(256) void q2_roundtrip_kernel(const float* __restrict__ w, int64_t n_blocks,
                                                           float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= n_blocks) return;  // uniform per wavefront
  const int64_t off = blk * kQK + 4 * lane;
  const float4 v = *reinterpret_cast<const float4*>(w + off);
  const float f[4] = {v.x, v.y, v.z, v.w};
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double a = static_cast<double>(f[j]);
    ss = (j == 0) ? a * a : ss + a * a;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss = ss + __shfl_xor(ss, m, 64);
  double s = sqrt(ss / 256.0) / 2.0;
  s = (s > 65504.0) ? 65504.0 : s;  // NaN passes through
  const float s32 = static_cast<float>(static_cast<_Float16>(static_cast<float>(s)));
  const float lo = s32, hi = 3.0f * s32;   // both exact in fp32
  float o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mag = (fabsf(f[j]) < 2.0f * s32) ? lo : hi;
    o[j] = __uint_as_float(__float_as_uint(mag) | (__float_as_uint(f[j]) & 0x80000000u));
  }
  *reinterpret_cast<float4*>(out + off) = make_float4(o[0], o[1], o[2], o[3]);
}

}  // namespace

// calibration tiles of the launch; one tile (of zeros) when there are no
// calibration rows, so the diagonal pass still runs
static int64_t cal_tiles(int64_t n_cal) { return n_cal > 0 ? (n_cal + kSensCal - 1) / kSensCal : 1; }

int64_t layer_errors_scratch_bytes(int64_t n_rows, int64_t k, int64_t n_cal) {
  const int64_t ctiles = cal_tiles(n_cal);
  return (k + 2 * ctiles * n_rows) * static_cast<int64_t>(sizeof(double));
}

hipError_t launch_layer_errors(const float* w, const float* w_hat, int64_t n_rows, int64_t k, const float* x,
                               int64_t n_cal, double* err_full, double* err_diag, void* scratch, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  double* hd = static_cast<double*>(scratch);
  double* partial = hd + k;
  const int rtiles = static_cast<int>((n_rows + kSensRows - 1) / kSensRows);
  const int ctiles = static_cast<int>(cal_tiles(n_cal));
  hipLaunchKernelGGL(hdiag_kernel, dim3(static_cast<unsigned>((k + kHdCols - 1) / kHdCols)), dim3(256), 0, s, x, n_cal,
                     k, hd);
  const int64_t groups = (rtiles + 7) / 8;
  hipLaunchKernelGGL(layer_errors_kernel, dim3(static_cast<unsigned>(groups * 8 * ctiles)), dim3(256), 0, s, w,
                     w_hat, static_cast<int>(n_rows), k, x, static_cast<int>(n_cal), hd, partial, err_diag, ctiles);
  hipLaunchKernelGGL(sum_partials_kernel, dim3(static_cast<unsigned>((n_rows + 255) / 256)), dim3(256), 0, s,
                     partial, 2 * ctiles, static_cast<int>(n_rows), err_full);
  return hipGetLastError();
}

hipError_t launch_q2_roundtrip(const float* w, int64_t n_rows, int64_t k, float* out, hipStream_t s) {
  const int64_t n_blocks = n_rows * (k / kQK);
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(q2_roundtrip_kernel, dim3(static_cast<unsigned>((n_blocks + 3) / 4)), dim3(256), 0, s, w,
                     n_blocks, out);
  return hipGetLastError();
}

}  // namespace stq
