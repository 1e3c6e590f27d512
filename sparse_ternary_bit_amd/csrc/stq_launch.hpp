// Host-side launchers of the libstq kernels (internal to the library).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stq {

hipError_t launch_dequantize(const uint8_t* q, int64_t n_rows, int64_t k, float* out, hipStream_t s);

hipError_t launch_quantize(const float* w, const float* imatrix, int64_t n_rows, int64_t k, int encoder,
                           int rounds, uint8_t* out, hipStream_t s);

struct GemvArgs {
  const uint8_t* w_table;
  int64_t expert_stride;
  int64_t n_experts;
  int64_t n;
  int64_t k;
  const void* x;
  int x_mode;               // 0 fp32 rows, 1 bf16 rows
  int64_t x_row_stride;     // elements
  int64_t n_tokens;
  const int32_t* pair_expert;
  const int32_t* pair_token;  // NULL: pair q uses token q / pairs_per_token
  int64_t n_pairs;
  float* y;
  int64_t pairs_per_token;  // used only without pair_token (0 means 1)
};

// Scratch needed by launch_gemv for the chosen k split (bytes, 0 if none),
// and the launch itself; with partial_bytes > 0, `partial` holds that many
// bytes (fp32 partial sums, then one int per pair).
struct GemvPlan {
  int splits;          // k split across workgroups
  int blocks_per_split;
  int max_sub;         // most parts a split's blocks are cut into for a many-token expert
  int64_t partial_floats;
  int64_t partial_bytes;
  bool mfma;           // bf16 passes of 3+ tokens on the matrix cores (kernel variant)
  bool order_units;    // more workgroups than resident slots: number units longest first
};
// cus: compute units the plan is made for (see cus_of_stream).
GemvPlan plan_gemv(const GemvArgs& a, int cus);
// Compute units of the device a stream runs on, or of the current device
// (256 when the query fails); cached per device.
int cus_of_stream(hipStream_t s);
int cus_of_current_device();
// reduce = false leaves split outputs in `partial` for the caller to add (see
// GemvPartials); the GEMV still writes y's rows that are not split and the
// NaN rows of invalid pairs.
hipError_t launch_gemv(const GemvArgs& a, const GemvPlan& plan, void* partial, hipStream_t s, bool reduce = true);

// Split outputs of a launch_gemv(..., reduce = false): valid pair p's row r
// is, when its slot count splits * (pair_sub ? pair_sub[p] : 1) exceeds 1,
// the sum over slots s in order, starting from 0.0f, of
// partial[(s * n_pairs + p) * n + r]; otherwise y's own row.  partial is
// NULL when the plan splits nothing.
struct GemvPartials {
  const float* partial;
  int splits;
  int max_slots;  // splits x the part cap: no pair has more slots
  const int32_t* pair_sub;
};
GemvPartials gemv_partials(const GemvPlan& plan, void* partial);

// h[p, c] = silu(gu[p, c]) * gu[p, d_ff + c], silu(v) = v / (1 + exp(-v)),
// for gu [n_pairs, 2*d_ff] and h [n_pairs, d_ff] fp32 (d_ff a multiple of 4),
// with gu the y of a launch_gemv(..., reduce = false) whose split rows are
// added here (pair_expert / n_experts tell valid pairs)
hipError_t launch_swiglu(const float* gu, const GemvPartials& parts, const int32_t* pair_expert, int64_t n_experts,
                         int64_t n_pairs, int64_t d_ff, float* h, hipStream_t s);

// y[t, :] = sum over k < top_k, in order, of w[t*top_k + k] * z[t*top_k + k, :],
// with z the y of a launch_gemv(..., reduce = false) over the pairs
hipError_t launch_combine(const float* z, const GemvPartials& parts, const int32_t* pair_expert, int64_t n_experts,
                          const float* w, int64_t n_tokens, int64_t top_k, int64_t n, float* y, hipStream_t s);

struct GemmArgs {
  const uint8_t* w_table;
  int64_t expert_stride;
  int64_t n_experts;
  int64_t n;
  int64_t k;
  const uint16_t* x;
  const int32_t* offsets;
  int64_t total_m;
  float* y;
};
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s);

// Layer error under calibration activations (full Hessian and diagonal);
// `scratch` holds layer_errors_scratch_bytes(...) bytes.
int64_t layer_errors_scratch_bytes(int64_t n_rows, int64_t k, int64_t n_cal);
hipError_t launch_layer_errors(const float* w, const float* w_hat, int64_t n_rows, int64_t k, const float* x,
                               int64_t n_cal, double* err_full, double* err_diag, void* scratch, hipStream_t s);

// 2-bit stand-in format: quantize and reconstruct in one pass
hipError_t launch_q2_roundtrip(const float* w, int64_t n_rows, int64_t k, float* out, hipStream_t s);

// Streaming-read reference (measurement only): reads `bytes` bytes of `buf`
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);

// Matrix-core and LDS references (measurement only).  Their shapes are the
// ones stq.h states, so that callers can count the work of a launch.
constexpr int kMfmaProbeGrid = 4096;  // workgroups of 4 wavefronts
constexpr int kMfmaChains = 8;        // independent MFMAs per wavefront and round
constexpr int kLdsProbeGrid = 4096;   // workgroups of 4 wavefronts
constexpr int kLdsReads = 8;          // LDS reads per wavefront and round
constexpr int kLdsProbeWords = 2048;  // 16-byte words of LDS per workgroup (32 KB)
hipError_t launch_mfma_loop(int64_t iters, float* sink, hipStream_t s);
hipError_t launch_lds_read(int mode, int64_t iters, uint32_t* sink, hipStream_t s);

}  // namespace stq
