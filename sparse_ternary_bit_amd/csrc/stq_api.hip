// C ABI of libstq: host-side validation, error reporting and dispatch.
// Every check runs before any HIP call, so a bad argument never reaches a
// kernel.  See include/stq.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "stq.h"
#include "stq_launch.hpp"

namespace {

thread_local std::string g_last_error;

stq_status fail(stq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

stq_status ok() {
  g_last_error.clear();
  return STQ_OK;
}

stq_status hip_fail(hipError_t e, const char* what) {
  return fail(STQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Caller-owned workspace: a call that needs `need` bytes accepts any buffer
// of at least that many bytes, 256-byte aligned (the kernels read partial
// sums 16 bytes at a time and sub-buffers start on 256-byte boundaries).
stq_status check_workspace(const void* ws, int64_t ws_bytes, int64_t need, const char* who) {
  if (ws_bytes < 0) return fail(STQ_E_ARG, "%s: workspace_bytes < 0", who);
  if (need <= 0) return STQ_OK;
  if (!ws || ws_bytes < need)
    return fail(STQ_E_ARG, "%s: needs a workspace of %lld bytes, got %lld%s", who, (long long)need,
                (long long)ws_bytes, ws ? "" : " (NULL)");
  if (!aligned(ws, 256)) return fail(STQ_E_ALIGN, "%s: workspace not 256-byte aligned", who);
  return STQ_OK;
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

extern "C" {

int64_t stq_row_bytes(int64_t k) {
  if (k <= 0 || k % STQ_QK != 0) return -1;
  return k / STQ_QK * STQ_BLOCK_BYTES;
}

const char* stq_status_string(stq_status s) {
  switch (s) {
    case STQ_OK: return "ok";
    case STQ_E_ARG: return "invalid argument";
    case STQ_E_SHAPE: return "invalid shape";
    case STQ_E_ALIGN: return "misaligned pointer or stride";
    case STQ_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* stq_last_error(void) { return g_last_error.c_str(); }

stq_status stq_quantize_rows(const float* w, const float* imatrix, int64_t n_rows, int64_t k, int encoder,
                             int rounds, uint8_t* out, stq_stream_t stream) {
  if (n_rows < 0) return fail(STQ_E_ARG, "stq_quantize_rows: n_rows < 0");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_quantize_rows: k=%lld is not a positive multiple of 256", (long long)k);
  if (encoder != STQ_ENC_WLS && encoder != STQ_ENC_AMAX) return fail(STQ_E_ARG, "stq_quantize_rows: unknown encoder %d", encoder);
  if (encoder == STQ_ENC_WLS && rounds < 0) return fail(STQ_E_ARG, "stq_quantize_rows: rounds < 0");
  if (n_rows > 0 && (!w || !out)) return fail(STQ_E_ARG, "stq_quantize_rows: null pointer");
  if (!aligned(w, 4) || !aligned(imatrix, 4)) return fail(STQ_E_ALIGN, "stq_quantize_rows: w/imatrix not 4-byte aligned");
  if (!aligned(out, 2)) return fail(STQ_E_ALIGN, "stq_quantize_rows: out not 2-byte aligned");
  if (n_rows > INT_MAX || k / STQ_QK > INT_MAX) return fail(STQ_E_SHAPE, "stq_quantize_rows: count exceeds int32");
  if (n_rows * (k / STQ_QK) > (int64_t)INT_MAX * 4) return fail(STQ_E_SHAPE, "stq_quantize_rows: too many blocks");
  hipError_t e = stq::launch_quantize(w, imatrix, n_rows, k, encoder, rounds, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_quantize_rows launch");
  return ok();
}

stq_status stq_dequantize_rows(const uint8_t* q, int64_t n_rows, int64_t k, float* out, stq_stream_t stream) {
  if (n_rows < 0) return fail(STQ_E_ARG, "stq_dequantize_rows: n_rows < 0");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_dequantize_rows: k=%lld is not a positive multiple of 256", (long long)k);
  if (n_rows > 0 && (!q || !out)) return fail(STQ_E_ARG, "stq_dequantize_rows: null pointer");
  if (!aligned(q, 2) || !aligned(out, 4)) return fail(STQ_E_ALIGN, "stq_dequantize_rows: q must be 2-byte and out 4-byte aligned");
  if (n_rows > INT_MAX || k / STQ_QK > INT_MAX) return fail(STQ_E_SHAPE, "stq_dequantize_rows: count exceeds int32");
  if (n_rows * (k / 4) > (int64_t)INT_MAX * 256) return fail(STQ_E_SHAPE, "stq_dequantize_rows: too many groups");
  hipError_t e = stq::launch_dequantize(q, n_rows, k, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_dequantize_rows launch");
  return ok();
}

namespace {

// Argument checks of stq_gemv and stq_gemv_noalloc; `nothing` is set when
// the call has no work (no pairs or no rows), which is not an error.
stq_status gemv_check(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts, int64_t n, int64_t k,
                      const void* x, int x_dtype, int64_t x_row_stride, int64_t n_tokens, const int32_t* pair_expert,
                      const int32_t* pair_token, int64_t n_pairs, const float* y, const char* who, bool* nothing) {
  *nothing = false;
  if (n_experts < 1 || n < 0 || n_tokens < 0 || n_pairs < 0) return fail(STQ_E_ARG, "%s: negative count or no experts", who);
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "%s: k=%lld is not a positive multiple of 256", who, (long long)k);
  if (x_dtype != STQ_X_F32 && x_dtype != STQ_X_BF16) return fail(STQ_E_ARG, "%s: unknown x_dtype %d", who, x_dtype);
  if (n > INT_MAX || n_tokens > INT_MAX || n_experts > INT_MAX) return fail(STQ_E_SHAPE, "%s: count exceeds int32", who);
  if (n_pairs > 65535) return fail(STQ_E_SHAPE, "%s: more than 65535 pairs in one call", who);
  const int64_t rb = stq_row_bytes(k);
  if (expert_stride_bytes < n * rb) return fail(STQ_E_SHAPE, "%s: expert stride %lld < n*row_bytes %lld", who, (long long)expert_stride_bytes, (long long)(n * rb));
  if (x_row_stride < k) return fail(STQ_E_SHAPE, "%s: x_row_stride < k", who);
  if (n_pairs == 0 || n == 0) {
    *nothing = true;
    return STQ_OK;
  }
  if (!w_table || !x || !y) return fail(STQ_E_ARG, "%s: null pointer", who);
  if (!aligned(w_table, 16) || expert_stride_bytes % 16) return fail(STQ_E_ALIGN, "%s: w_table / expert stride not 16-byte aligned", who);
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(pair_expert, 4) || !aligned(pair_token, 4)) return fail(STQ_E_ALIGN, "%s: x, y or pair arrays not 4-byte aligned", who);
  if (x_dtype == STQ_X_BF16 && (x_row_stride % 2)) return fail(STQ_E_ALIGN, "%s: bf16 x_row_stride must be even", who);
  return STQ_OK;
}

}  // namespace

stq_status stq_gemv(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts, int64_t n, int64_t k,
                    const void* x, int x_dtype, int64_t x_row_stride, int64_t n_tokens,
                    const int32_t* pair_expert, const int32_t* pair_token, int64_t n_pairs, float* y,
                    void* workspace, int64_t workspace_bytes, stq_stream_t stream) {
  bool nothing = false;
  stq_status st = gemv_check(w_table, expert_stride_bytes, n_experts, n, k, x, x_dtype, x_row_stride, n_tokens,
                             pair_expert, pair_token, n_pairs, y, "stq_gemv", &nothing);
  if (st != STQ_OK) return st;
  if (workspace_bytes < 0) return fail(STQ_E_ARG, "stq_gemv: workspace_bytes < 0");
  if (nothing) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  stq::GemvArgs ga{w_table, expert_stride_bytes, n_experts, n, k, x, x_dtype == STQ_X_BF16 ? 1 : 0,
                   x_row_stride, n_tokens, pair_expert, pair_token, n_pairs, y, 1};
  const stq::GemvPlan pl = stq::plan_gemv(ga, stq::cus_of_stream(s));
  st = check_workspace(workspace, workspace_bytes, pl.partial_bytes, "stq_gemv");
  if (st != STQ_OK) return st;
  hipError_t le = stq::launch_gemv(ga, pl, workspace, s);
  if (le != hipSuccess) return hip_fail(le, "stq_gemv launch");
  return ok();
}

stq_status stq_gemv_plan(int64_t n_experts, int64_t n, int64_t k, int64_t n_pairs, int32_t n_cus,
                         int32_t* splits, int32_t* max_parts, int64_t* scratch_bytes) {
  if (!splits || !max_parts || !scratch_bytes) return fail(STQ_E_ARG, "stq_gemv_plan: null output pointer");
  if (n_experts < 1 || n < 0 || n_pairs < 0 || n_cus < 0) return fail(STQ_E_ARG, "stq_gemv_plan: negative count or no experts");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_gemv_plan: k=%lld is not a positive multiple of 256", (long long)k);
  if (n > INT_MAX || n_experts > INT_MAX) return fail(STQ_E_SHAPE, "stq_gemv_plan: count exceeds int32");
  if (n_pairs > 65535) return fail(STQ_E_SHAPE, "stq_gemv_plan: more than 65535 pairs in one call");
  *splits = 1;
  *max_parts = 1;
  *scratch_bytes = 0;
  if (n_pairs == 0 || n == 0) return ok();  // stq_gemv launches nothing
  const stq::GemvArgs ga{nullptr, n * stq_row_bytes(k), n_experts, n, k, nullptr, 1, k, 1, nullptr, nullptr,
                         n_pairs, nullptr, 1};
  const stq::GemvPlan pl = stq::plan_gemv(ga, n_cus > 0 ? n_cus : stq::cus_of_current_device());
  *splits = pl.splits;
  *max_parts = pl.max_sub;
  *scratch_bytes = pl.partial_bytes;
  return ok();
}

namespace {

// Shape checks shared by stq_moe_ffn_decode and its workspace query.
stq_status ffn_shape_check(int64_t n_experts, int64_t d_model, int64_t d_ff, int64_t n_tokens, int64_t top_k,
                           const char* who) {
  if (n_experts < 1 || n_tokens < 0 || top_k < 1) return fail(STQ_E_ARG, "%s: bad count (n_experts >= 1, n_tokens >= 0, top_k >= 1)", who);
  if (d_model <= 0 || d_model % STQ_QK || d_ff <= 0 || d_ff % STQ_QK)
    return fail(STQ_E_SHAPE, "%s: d_model and d_ff must be positive multiples of 256", who);
  if (d_model > INT_MAX / 2 || 2 * d_ff > INT_MAX || n_experts > INT_MAX) return fail(STQ_E_SHAPE, "%s: size exceeds int32", who);
  if (n_tokens > 65535 / top_k) return fail(STQ_E_SHAPE, "%s: more than 65535 (token, expert) pairs", who);
  return STQ_OK;
}

// The FFN's workspace: the two GEMVs' split outputs (one region, reused),
// then the gate/up rows, the activations and the down projections' rows of
// every pair, each on a 256-byte boundary.
struct FfnLayout {
  stq::GemvArgs g1, g2;
  stq::GemvPlan p1, p2;
  int64_t part, gu, h, z, total;
};

FfnLayout ffn_layout(const uint8_t* w_gate_up, int64_t gate_up_stride_bytes, const uint8_t* w_down,
                     int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff, const uint16_t* x,
                     int64_t n_tokens, const int32_t* pair_expert, int64_t top_k, int cus) {
  FfnLayout L{};
  const int64_t P = n_tokens * top_k;
  L.g1 = stq::GemvArgs{w_gate_up, gate_up_stride_bytes, n_experts, 2 * d_ff, d_model, x, 1, d_model, n_tokens,
                       pair_expert, nullptr, P, nullptr, top_k};
  L.g2 = stq::GemvArgs{w_down, down_stride_bytes, n_experts, d_model, d_ff, nullptr, 0, d_ff, P,
                       pair_expert, nullptr, P, nullptr, 1};
  L.p1 = stq::plan_gemv(L.g1, cus);
  L.p2 = stq::plan_gemv(L.g2, cus);
  L.part = round256(std::max(L.p1.partial_bytes, L.p2.partial_bytes));
  L.gu = round256(P * 2 * d_ff * 4);
  L.h = round256(P * d_ff * 4);
  L.z = round256(P * d_model * 4);
  L.total = P == 0 ? 0 : L.part + L.gu + L.h + L.z;
  return L;
}

}  // namespace

stq_status stq_moe_ffn_workspace(int64_t n_experts, int64_t d_model, int64_t d_ff, int64_t n_tokens, int64_t top_k,
                                 int32_t n_cus, int64_t* workspace_bytes) {
  if (!workspace_bytes) return fail(STQ_E_ARG, "stq_moe_ffn_workspace: null output pointer");
  *workspace_bytes = 0;
  if (n_cus < 0) return fail(STQ_E_ARG, "stq_moe_ffn_workspace: n_cus < 0");
  const stq_status st = ffn_shape_check(n_experts, d_model, d_ff, n_tokens, top_k, "stq_moe_ffn_workspace");
  if (st != STQ_OK) return st;
  const FfnLayout L = ffn_layout(nullptr, 2 * d_ff * stq_row_bytes(d_model), nullptr, d_model * stq_row_bytes(d_ff),
                                 n_experts, d_model, d_ff, nullptr, n_tokens, nullptr, top_k,
                                 n_cus > 0 ? n_cus : stq::cus_of_current_device());
  *workspace_bytes = L.total;
  return ok();
}

stq_status stq_moe_ffn_decode(const uint8_t* w_gate_up, int64_t gate_up_stride_bytes, const uint8_t* w_down,
                              int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
                              const uint16_t* x, int64_t n_tokens, const int32_t* pair_expert,
                              const float* pair_weight, int64_t top_k, float* y, void* workspace,
                              int64_t workspace_bytes, stq_stream_t stream) {
  const stq_status sc = ffn_shape_check(n_experts, d_model, d_ff, n_tokens, top_k, "stq_moe_ffn_decode");
  if (sc != STQ_OK) return sc;
  if (gate_up_stride_bytes < 2 * d_ff * stq_row_bytes(d_model) || down_stride_bytes < d_model * stq_row_bytes(d_ff))
    return fail(STQ_E_SHAPE, "stq_moe_ffn_decode: expert stride smaller than the packed matrix");
  if (workspace_bytes < 0) return fail(STQ_E_ARG, "stq_moe_ffn_decode: workspace_bytes < 0");
  if (n_tokens == 0) return ok();
  if (!w_gate_up || !w_down || !x || !pair_expert || !pair_weight || !y) return fail(STQ_E_ARG, "stq_moe_ffn_decode: null pointer");
  if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || gate_up_stride_bytes % 16 || down_stride_bytes % 16)
    return fail(STQ_E_ALIGN, "stq_moe_ffn_decode: tables / strides not 16-byte aligned");
  if (!aligned(x, 4) || !aligned(pair_expert, 4) || !aligned(pair_weight, 4) || !aligned(y, 4))
    return fail(STQ_E_ALIGN, "stq_moe_ffn_decode: x, pair arrays or y not 4-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  FfnLayout L = ffn_layout(w_gate_up, gate_up_stride_bytes, w_down, down_stride_bytes, n_experts, d_model, d_ff, x,
                           n_tokens, pair_expert, top_k, stq::cus_of_stream(s));
  const stq_status st = check_workspace(workspace, workspace_bytes, L.total, "stq_moe_ffn_decode");
  if (st != STQ_OK) return st;
  const int64_t P = n_tokens * top_k;
  char* b = static_cast<char*>(workspace);
  float* gu = reinterpret_cast<float*>(b + L.part);
  float* h = reinterpret_cast<float*>(b + L.part + L.gu);
  float* z = reinterpret_cast<float*>(b + L.part + L.gu + L.h);
  L.g1.y = gu;
  L.g2.x = h;
  L.g2.y = z;
  // gate/up GEMV of every pair's token, SwiGLU of each gate/up row, then the
  // down GEMV of every pair's activation row; each GEMV's split outputs are
  // added by the next step (SwiGLU, combine) instead of a reduction launch of
  // its own, in the same order
  hipError_t e = stq::launch_gemv(L.g1, L.p1, b, s, false);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: gate/up launch");
  e = stq::launch_swiglu(gu, stq::gemv_partials(L.p1, b), pair_expert, n_experts, P, d_ff, h, s);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: SwiGLU launch");
  e = stq::launch_gemv(L.g2, L.p2, b, s, false);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: down launch");
  e = stq::launch_combine(z, stq::gemv_partials(L.p2, b), pair_expert, n_experts, pair_weight, n_tokens, top_k,
                          d_model, y, s);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: combine launch");
  return ok();
}

stq_status stq_grouped_gemm(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts, int64_t n,
                            int64_t k, const uint16_t* x_sorted, const int32_t* expert_offsets, int64_t total_m,
                            float* y, stq_stream_t stream) {
  if (n_experts < 1 || n < 0 || total_m < 0) return fail(STQ_E_ARG, "stq_grouped_gemm: negative count or no experts");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_grouped_gemm: k=%lld is not a positive multiple of 256", (long long)k);
  if (n > INT_MAX || total_m > INT_MAX) return fail(STQ_E_SHAPE, "stq_grouped_gemm: count exceeds int32");
  if (n_experts > 65535) return fail(STQ_E_SHAPE, "stq_grouped_gemm: more than 65535 experts");
  const int64_t rb = stq_row_bytes(k);
  if (expert_stride_bytes < n * rb) return fail(STQ_E_SHAPE, "stq_grouped_gemm: expert stride < n*row_bytes");
  if (!expert_offsets) return fail(STQ_E_ARG, "stq_grouped_gemm: null offsets");
  if (total_m == 0 || n == 0) return ok();
  if (!w_table || !x_sorted || !y) return fail(STQ_E_ARG, "stq_grouped_gemm: null pointer");
  if (!aligned(w_table, 16) || expert_stride_bytes % 16) return fail(STQ_E_ALIGN, "stq_grouped_gemm: w_table / expert stride not 16-byte aligned");
  if (!aligned(x_sorted, 16)) return fail(STQ_E_ALIGN, "stq_grouped_gemm: x_sorted not 16-byte aligned");
  if (!aligned(expert_offsets, 4) || !aligned(y, 4)) return fail(STQ_E_ALIGN, "stq_grouped_gemm: offsets / y not 4-byte aligned");
  stq::GemmArgs ga{w_table, expert_stride_bytes, n_experts, n, k, x_sorted, expert_offsets, total_m, y};
  hipError_t e = stq::launch_grouped_gemm(ga, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_grouped_gemm launch");
  return ok();
}

namespace {

stq_status layer_errors_shape_check(int64_t n_rows, int64_t k, int64_t n_calib, const char* who) {
  if (n_rows < 0) return fail(STQ_E_ARG, "%s: n_rows < 0", who);
  if (n_calib < 1) return fail(STQ_E_ARG, "%s: n_calib must be >= 1", who);
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "%s: k=%lld is not a positive multiple of 256", who, (long long)k);
  if (n_rows > INT_MAX || n_calib > INT_MAX) return fail(STQ_E_SHAPE, "%s: count exceeds int32", who);
  if ((n_calib + 63) / 64 > 65535) return fail(STQ_E_SHAPE, "%s: more than 65535*64 calibration rows", who);
  if (((n_rows + 511) / 512) * 8 * ((n_calib + 63) / 64) > INT_MAX) return fail(STQ_E_SHAPE, "%s: too many tiles", who);
  return STQ_OK;
}

}  // namespace

stq_status stq_layer_errors_workspace(int64_t n_rows, int64_t k, int64_t n_calib, int64_t* workspace_bytes) {
  if (!workspace_bytes) return fail(STQ_E_ARG, "stq_layer_errors_workspace: null output pointer");
  *workspace_bytes = 0;
  const stq_status st = layer_errors_shape_check(n_rows, k, n_calib, "stq_layer_errors_workspace");
  if (st != STQ_OK) return st;
  *workspace_bytes = n_rows == 0 ? 0 : stq::layer_errors_scratch_bytes(n_rows, k, n_calib);
  return ok();
}

stq_status stq_layer_errors(const float* w, const float* w_hat, int64_t n_rows, int64_t k, const float* x_calib,
                            int64_t n_calib, double* err_full, double* err_diag, void* workspace,
                            int64_t workspace_bytes, stq_stream_t stream) {
  const stq_status sc = layer_errors_shape_check(n_rows, k, n_calib, "stq_layer_errors");
  if (sc != STQ_OK) return sc;
  if (workspace_bytes < 0) return fail(STQ_E_ARG, "stq_layer_errors: workspace_bytes < 0");
  if (n_rows == 0) return ok();
  if (!w || !w_hat || !x_calib || !err_full || !err_diag) return fail(STQ_E_ARG, "stq_layer_errors: null pointer");
  if (!aligned(w, 16) || !aligned(w_hat, 16) || !aligned(x_calib, 16))
    return fail(STQ_E_ALIGN, "stq_layer_errors: w, w_hat and x_calib must be 16-byte aligned");
  if (!aligned(err_full, 8) || !aligned(err_diag, 8)) return fail(STQ_E_ALIGN, "stq_layer_errors: outputs not 8-byte aligned");
  const stq_status st = check_workspace(workspace, workspace_bytes, stq::layer_errors_scratch_bytes(n_rows, k, n_calib),
                                        "stq_layer_errors");
  if (st != STQ_OK) return st;
  hipError_t e = stq::launch_layer_errors(w, w_hat, n_rows, k, x_calib, n_calib, err_full, err_diag, workspace,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_layer_errors launch");
  return ok();
}

stq_status stq_q2_roundtrip(const float* w, int64_t n_rows, int64_t k, float* out, stq_stream_t stream) {
  if (n_rows < 0) return fail(STQ_E_ARG, "stq_q2_roundtrip: n_rows < 0");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_q2_roundtrip: k=%lld is not a positive multiple of 256", (long long)k);
  if (n_rows > INT_MAX || n_rows * (k / STQ_QK) > (int64_t)INT_MAX * 4) return fail(STQ_E_SHAPE, "stq_q2_roundtrip: too many blocks");
  if (n_rows == 0) return ok();
  if (!w || !out) return fail(STQ_E_ARG, "stq_q2_roundtrip: null pointer");
  if (!aligned(w, 16) || !aligned(out, 16)) return fail(STQ_E_ALIGN, "stq_q2_roundtrip: w and out must be 16-byte aligned");
  hipError_t e = stq::launch_q2_roundtrip(w, n_rows, k, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_q2_roundtrip launch");
  return ok();
}

stq_status stq_greedy_allocation(const double* gain, const double* extra_bytes, int64_t n_layers, double budget,
                                 uint8_t* chosen) {
  if (n_layers < 0) return fail(STQ_E_ARG, "stq_greedy_allocation: n_layers < 0");
  if (n_layers == 0) return ok();
  if (!gain || !extra_bytes || !chosen) return fail(STQ_E_ARG, "stq_greedy_allocation: null pointer");
  for (int64_t i = 0; i < n_layers; ++i)
    if (!(extra_bytes[i] > 0.0)) return fail(STQ_E_ARG, "stq_greedy_allocation: extra_bytes[%lld] must be > 0", (long long)i);
  std::vector<int64_t> order(static_cast<size_t>(n_layers));
  std::vector<double> ratio(static_cast<size_t>(n_layers));
  for (int64_t i = 0; i < n_layers; ++i) {
    order[i] = i;
    ratio[i] = gain[i] / extra_bytes[i];
  }
  // largest reduction per added byte first, lowest index on ties
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return ratio[a] > ratio[b]; });
  double used = 0.0;
  for (int64_t i = 0; i < n_layers; ++i) chosen[i] = 0;
  for (int64_t i : order) {
    if (gain[i] > 0.0 && used + extra_bytes[i] <= budget) {
      chosen[i] = 1;
      used += extra_bytes[i];
    }
  }
  return ok();
}

stq_status stq_stream_read_probe(const void* buf, int64_t bytes, uint32_t* sink, stq_stream_t stream) {
  if (bytes < 0 || bytes % 16) return fail(STQ_E_ARG, "stq_stream_read_probe: bytes must be a non-negative multiple of 16");
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(STQ_E_ARG, "stq_stream_read_probe: null pointer");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(STQ_E_ALIGN, "stq_stream_read_probe: buf must be 16-byte and sink 4-byte aligned");
  hipError_t e = stq::launch_stream_read(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_stream_read_probe launch");
  return ok();
}

static_assert(STQ_MFMA_PROBE_FLOP_PER_ROUND == 4.0 * stq::kMfmaProbeGrid * stq::kMfmaChains * 16384.0,
              "the MFMA probe's stated work per round");
static_assert(STQ_LDS_PROBE_READS_PER_ROUND == 4 * stq::kLdsProbeGrid * stq::kLdsReads,
              "the LDS probe's stated reads per round");

stq_status stq_mfma_loop_probe(int64_t rounds, float* sink, stq_stream_t stream) {
  if (rounds < 0) return fail(STQ_E_ARG, "stq_mfma_loop_probe: rounds must be >= 0");
  if (rounds == 0) return ok();
  if (!sink) return fail(STQ_E_ARG, "stq_mfma_loop_probe: null sink");
  if (!aligned(sink, 4)) return fail(STQ_E_ALIGN, "stq_mfma_loop_probe: sink must be 4-byte aligned");
  hipError_t e = stq::launch_mfma_loop(rounds, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_mfma_loop_probe launch");
  return ok();
}

stq_status stq_lds_read_probe(int mode, int64_t rounds, uint32_t* sink, stq_stream_t stream) {
  if (mode != 0 && mode != 1) return fail(STQ_E_ARG, "stq_lds_read_probe: mode must be 0 or 1");
  if (rounds < 0) return fail(STQ_E_ARG, "stq_lds_read_probe: rounds must be >= 0");
  if (rounds == 0) return ok();
  if (!sink) return fail(STQ_E_ARG, "stq_lds_read_probe: null sink");
  if (!aligned(sink, 4)) return fail(STQ_E_ALIGN, "stq_lds_read_probe: sink must be 4-byte aligned");
  hipError_t e = stq::launch_lds_read(mode, rounds, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stq_lds_read_probe launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// stq_gemv_noalloc: stq_gemv for callers that cannot allocate.  Its split
// outputs live in `scratch`, a fixed array of device memory in the library
// itself (each GPU holds its own copy from the library's load until the
// process ends).  In host code `scratch` names a host-side stand-in, so the
// device address of each GPU's copy is looked up once per device with that
// device current and kept; only that address reaches a kernel.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kNoAllocScratchBytes = STQ_GEMV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

stq_status scratch_for_stream(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return hip_fail(e, "stq_gemv_noalloc: device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(STQ_E_HIP, "stq_gemv_noalloc: device %d out of range", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return hip_fail(e, "stq_gemv_noalloc: current device");
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "stq_gemv_noalloc: set device");
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return hip_fail(e, "stq_gemv_noalloc: scratch address");
      if (back != hipSuccess) return hip_fail(back, "stq_gemv_noalloc: restore device");
      if (!q || !aligned(q, 256)) return fail(STQ_E_HIP, "stq_gemv_noalloc: scratch address unusable");
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return STQ_OK;
}

}  // namespace

extern "C" {

stq_status stq_gemv_noalloc(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts, int64_t n,
                            int64_t k, const void* x, int x_dtype, int64_t x_row_stride, int64_t n_tokens,
                            const int32_t* pair_expert, const int32_t* pair_token, int64_t n_pairs, float* y,
                            stq_stream_t stream) {
  bool nothing = false;
  stq_status st = gemv_check(w_table, expert_stride_bytes, n_experts, n, k, x, x_dtype, x_row_stride, n_tokens,
                             pair_expert, pair_token, n_pairs, y, "stq_gemv_noalloc", &nothing);
  if (st != STQ_OK || nothing) return st == STQ_OK ? ok() : st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  stq::GemvArgs ga{w_table, expert_stride_bytes, n_experts, n, k, x, x_dtype == STQ_X_BF16 ? 1 : 0,
                   x_row_stride, n_tokens, pair_expert, pair_token, n_pairs, y, 1};
  const stq::GemvPlan pl = stq::plan_gemv(ga, stq::cus_of_stream(s));
  if (pl.partial_bytes > kNoAllocScratchBytes)
    return fail(STQ_E_SHAPE, "stq_gemv_noalloc: these shapes need %lld bytes of scratch, more than the %lld it holds",
                (long long)pl.partial_bytes, (long long)kNoAllocScratchBytes);
  void* ws = nullptr;
  if (pl.partial_bytes > 0) {
    st = scratch_for_stream(s, &ws);
    if (st != STQ_OK) return st;
  }
  hipError_t le = stq::launch_gemv(ga, pl, ws, s);
  if (le != hipSuccess) return hip_fail(le, "stq_gemv_noalloc launch");
  return ok();
}

}  // extern "C"
