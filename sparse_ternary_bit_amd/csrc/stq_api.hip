// C ABI of libstq: host-side validation, error reporting and dispatch.
// Every check runs before any HIP call, so a bad argument never reaches a
// kernel.  See include/stq.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>
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

// Per-device scratch arena for split-k partial sums and the FFN's
// intermediates: grown with hipMalloc when a call needs more (hipFree of the
// old arena waits for work that may still use it) and kept until the
// process ends.
struct Arena {
  void* ptr = nullptr;
  int64_t cap = 0;
};
std::mutex g_arena_mu;
std::unordered_map<int, Arena> g_arena;

stq_status arena_get(int64_t bytes, void** out, const char* who) {
  *out = nullptr;
  if (bytes <= 0) return STQ_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, who);
  std::lock_guard<std::mutex> lk(g_arena_mu);
  Arena& a = g_arena[dev];
  if (a.cap < bytes) {
    if (a.ptr) {
      e = hipFree(a.ptr);
      a.ptr = nullptr;
      a.cap = 0;
      if (e != hipSuccess) return hip_fail(e, who);
    }
    void* p = nullptr;
    e = hipMalloc(&p, static_cast<size_t>(bytes));
    if (e != hipSuccess) return hip_fail(e, who);
    a.ptr = p;
    a.cap = bytes;
  }
  *out = a.ptr;
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

stq_status stq_gemv(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts, int64_t n, int64_t k,
                    const void* x, int x_dtype, int64_t x_row_stride, int64_t n_tokens,
                    const int32_t* pair_expert, const int32_t* pair_token, int64_t n_pairs, float* y,
                    stq_stream_t stream) {
  if (n_experts < 1 || n < 0 || n_tokens < 0 || n_pairs < 0) return fail(STQ_E_ARG, "stq_gemv: negative count or no experts");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_gemv: k=%lld is not a positive multiple of 256", (long long)k);
  if (x_dtype != STQ_X_F32 && x_dtype != STQ_X_BF16) return fail(STQ_E_ARG, "stq_gemv: unknown x_dtype %d", x_dtype);
  if (n > INT_MAX || n_tokens > INT_MAX || n_experts > INT_MAX) return fail(STQ_E_SHAPE, "stq_gemv: count exceeds int32");
  if (n_pairs > 65535) return fail(STQ_E_SHAPE, "stq_gemv: more than 65535 pairs in one call");
  const int64_t rb = stq_row_bytes(k);
  if (expert_stride_bytes < n * rb) return fail(STQ_E_SHAPE, "stq_gemv: expert stride %lld < n*row_bytes %lld", (long long)expert_stride_bytes, (long long)(n * rb));
  if (x_row_stride < k) return fail(STQ_E_SHAPE, "stq_gemv: x_row_stride < k");
  if (n_pairs == 0 || n == 0) return ok();
  if (!w_table || !x || !y) return fail(STQ_E_ARG, "stq_gemv: null pointer");
  if (!aligned(w_table, 16) || expert_stride_bytes % 16) return fail(STQ_E_ALIGN, "stq_gemv: w_table / expert stride not 16-byte aligned");
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(pair_expert, 4) || !aligned(pair_token, 4)) return fail(STQ_E_ALIGN, "stq_gemv: x, y or pair arrays not 4-byte aligned");
  if (x_dtype == STQ_X_BF16 && (x_row_stride % 2)) return fail(STQ_E_ALIGN, "stq_gemv: bf16 x_row_stride must be even");

  stq::GemvArgs ga{w_table, expert_stride_bytes, n_experts, n, k, x, x_dtype == STQ_X_BF16 ? 1 : 0,
                   x_row_stride, n_tokens, pair_expert, pair_token, n_pairs, y, 1};
  const stq::GemvPlan pl = stq::plan_gemv(ga);
  void* partial = nullptr;
  const stq_status st = arena_get(pl.partial_bytes, &partial, "stq_gemv: scratch");
  if (st != STQ_OK) return st;
  hipError_t le = stq::launch_gemv(ga, pl, partial, reinterpret_cast<hipStream_t>(stream));
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
  const stq::GemvPlan pl = stq::plan_gemv(ga, n_cus);
  *splits = pl.splits;
  *max_parts = pl.max_sub;
  *scratch_bytes = pl.partial_bytes;
  return ok();
}

stq_status stq_moe_ffn_decode(const uint8_t* w_gate_up, int64_t gate_up_stride_bytes, const uint8_t* w_down,
                              int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
                              const uint16_t* x, int64_t n_tokens, const int32_t* pair_expert,
                              const float* pair_weight, int64_t top_k, float* y, stq_stream_t stream) {
  if (n_experts < 1 || n_tokens < 0 || top_k < 1) return fail(STQ_E_ARG, "stq_moe_ffn_decode: bad count (n_experts >= 1, n_tokens >= 0, top_k >= 1)");
  if (d_model <= 0 || d_model % STQ_QK || d_ff <= 0 || d_ff % STQ_QK)
    return fail(STQ_E_SHAPE, "stq_moe_ffn_decode: d_model and d_ff must be positive multiples of 256");
  if (d_model > INT_MAX / 2 || 2 * d_ff > INT_MAX || n_experts > INT_MAX) return fail(STQ_E_SHAPE, "stq_moe_ffn_decode: size exceeds int32");
  if (n_tokens > 65535 / top_k) return fail(STQ_E_SHAPE, "stq_moe_ffn_decode: more than 65535 (token, expert) pairs");
  if (gate_up_stride_bytes < 2 * d_ff * stq_row_bytes(d_model) || down_stride_bytes < d_model * stq_row_bytes(d_ff))
    return fail(STQ_E_SHAPE, "stq_moe_ffn_decode: expert stride smaller than the packed matrix");
  if (n_tokens == 0) return ok();
  if (!w_gate_up || !w_down || !x || !pair_expert || !pair_weight || !y) return fail(STQ_E_ARG, "stq_moe_ffn_decode: null pointer");
  if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || gate_up_stride_bytes % 16 || down_stride_bytes % 16)
    return fail(STQ_E_ALIGN, "stq_moe_ffn_decode: tables / strides not 16-byte aligned");
  if (!aligned(x, 4) || !aligned(pair_expert, 4) || !aligned(pair_weight, 4) || !aligned(y, 4))
    return fail(STQ_E_ALIGN, "stq_moe_ffn_decode: x, pair arrays or y not 4-byte aligned");

  const int64_t P = n_tokens * top_k;
  // gate/up GEMV of every pair's token, SwiGLU of each gate/up row, then the
  // down GEMV of every pair's activation row
  stq::GemvArgs g1{w_gate_up, gate_up_stride_bytes, n_experts, 2 * d_ff, d_model, x, 1, d_model, n_tokens,
                   pair_expert, nullptr, P, nullptr, top_k};
  stq::GemvArgs g2{w_down, down_stride_bytes, n_experts, d_model, d_ff, nullptr, 0, d_ff, P,
                   pair_expert, nullptr, P, nullptr, 1};
  const stq::GemvPlan p1 = stq::plan_gemv(g1), p2 = stq::plan_gemv(g2);
  const int64_t part = round256(std::max(p1.partial_bytes, p2.partial_bytes));
  const int64_t gu_bytes = round256(P * 2 * d_ff * 4);
  const int64_t h_bytes = round256(P * d_ff * 4);
  const int64_t z_bytes = round256(P * d_model * 4);
  void* base = nullptr;
  const stq_status st = arena_get(part + gu_bytes + h_bytes + z_bytes, &base, "stq_moe_ffn_decode: scratch");
  if (st != STQ_OK) return st;
  char* b = static_cast<char*>(base);
  float* gu = reinterpret_cast<float*>(b + part);
  float* h = reinterpret_cast<float*>(b + part + gu_bytes);
  float* z = reinterpret_cast<float*>(b + part + gu_bytes + h_bytes);
  g1.y = gu;
  g2.x = h;
  g2.y = z;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // each GEMV's split outputs are added by the next step (SwiGLU, combine)
  // instead of a reduction launch of its own; the order of the adds is the same
  hipError_t e = stq::launch_gemv(g1, p1, b, s, false);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: gate/up launch");
  e = stq::launch_swiglu(gu, stq::gemv_partials(p1, b), pair_expert, n_experts, P, d_ff, h, s);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: SwiGLU launch");
  e = stq::launch_gemv(g2, p2, b, s, false);
  if (e != hipSuccess) return hip_fail(e, "stq_moe_ffn_decode: down launch");
  e = stq::launch_combine(z, stq::gemv_partials(p2, b), pair_expert, n_experts, pair_weight, n_tokens, top_k,
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

stq_status stq_layer_errors(const float* w, const float* w_hat, int64_t n_rows, int64_t k, const float* x_calib,
                            int64_t n_calib, double* err_full, double* err_diag, stq_stream_t stream) {
  if (n_rows < 0) return fail(STQ_E_ARG, "stq_layer_errors: n_rows < 0");
  if (n_calib < 1) return fail(STQ_E_ARG, "stq_layer_errors: n_calib must be >= 1");
  if (k <= 0 || k % STQ_QK) return fail(STQ_E_SHAPE, "stq_layer_errors: k=%lld is not a positive multiple of 256", (long long)k);
  if (n_rows > INT_MAX || n_calib > INT_MAX) return fail(STQ_E_SHAPE, "stq_layer_errors: count exceeds int32");
  if ((n_calib + 63) / 64 > 65535) return fail(STQ_E_SHAPE, "stq_layer_errors: more than 65535*64 calibration rows");
  if (((n_rows + 511) / 512) * 8 * ((n_calib + 63) / 64) > INT_MAX) return fail(STQ_E_SHAPE, "stq_layer_errors: too many tiles");
  if (n_rows == 0) return ok();
  if (!w || !w_hat || !x_calib || !err_full || !err_diag) return fail(STQ_E_ARG, "stq_layer_errors: null pointer");
  if (!aligned(w, 16) || !aligned(w_hat, 16) || !aligned(x_calib, 16))
    return fail(STQ_E_ALIGN, "stq_layer_errors: w, w_hat and x_calib must be 16-byte aligned");
  if (!aligned(err_full, 8) || !aligned(err_diag, 8)) return fail(STQ_E_ALIGN, "stq_layer_errors: outputs not 8-byte aligned");
  void* scratch = nullptr;
  const stq_status st = arena_get(stq::layer_errors_scratch_bytes(n_rows, k, n_calib), &scratch, "stq_layer_errors: scratch");
  if (st != STQ_OK) return st;
  hipError_t e = stq::launch_layer_errors(w, w_hat, n_rows, k, x_calib, n_calib, err_full, err_diag, scratch,
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

}  // extern "C"
