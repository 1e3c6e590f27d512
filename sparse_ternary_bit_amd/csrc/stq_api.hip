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

// Per-device scratch of stq_gemv: [counters | partial sums].  The counter
// part is zeroed when allocated and the kernels leave it zeroed.
struct Scratch {
  void* ptr = nullptr;
  int64_t counter_cap = 0;
  int64_t partial_cap = 0;
};
std::mutex g_scratch_mu;
std::unordered_map<int, Scratch> g_scratch;

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
                   x_row_stride, n_tokens, pair_expert, pair_token, n_pairs, y};
  const stq::GemvPlan pl = stq::plan_gemv(ga);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (pl.splits > 1) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "stq_gemv: hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    Scratch& sc = g_scratch[dev];
    if (sc.counter_cap < pl.counter_bytes || sc.partial_cap < pl.partial_bytes) {
      const int64_t cc = std::max(sc.counter_cap, pl.counter_bytes);
      const int64_t pc = std::max(sc.partial_cap, pl.partial_bytes);
      if (sc.ptr) {
        e = hipFree(sc.ptr);  // waits for work that may still use it
        sc.ptr = nullptr;
        sc.counter_cap = sc.partial_cap = 0;
        if (e != hipSuccess) return hip_fail(e, "stq_gemv: hipFree scratch");
      }
      void* p = nullptr;
      e = hipMalloc(&p, static_cast<size_t>(cc + pc));
      if (e != hipSuccess) return hip_fail(e, "stq_gemv: hipMalloc scratch");
      e = hipMemset(p, 0, static_cast<size_t>(cc));
      if (e != hipSuccess) {
        (void)hipFree(p);
        return hip_fail(e, "stq_gemv: zeroing scratch counters");
      }
      sc.ptr = p;
      sc.counter_cap = cc;
      sc.partial_cap = pc;
    }
    scratch = sc.ptr;
    hipError_t le = stq::launch_gemv(ga, pl, static_cast<char*>(scratch), static_cast<char*>(scratch) + sc.counter_cap, s);
    if (le != hipSuccess) return hip_fail(le, "stq_gemv launch");
    return ok();
  }
  hipError_t le = stq::launch_gemv(ga, pl, nullptr, nullptr, s);
  if (le != hipSuccess) return hip_fail(le, "stq_gemv launch");
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

}  // extern "C"
