/*
 * stq.h -- C ABI of libstq, the STQ1_0 sparse-ternary quantized matmul for
 * AMD Instinct MI355X (gfx950).
 *
 * STQ1_0 (sources named by page title / address and section):
 *   - every group of four consecutive weights holds values in {-d, 0, +d} with
 *     exactly one zero lane: 4 zero positions x 8 sign choices = 32 patterns,
 *     five bits per group (lemmy.durstig.online post 66506, paragraph "Four
 *     weights, five bits");
 *   - the five bits are a 4-bit code plus a 1-bit table select into a
 *     32-entry codebook, one fp16 scale d is shared by 256 weights, and a block
 *     of 256 weights takes 42 bytes, 1.3125 bits per weight (alphasignal.ai,
 *     "AngelSlim Shrinks Tencent's 1.5TB Hy4-Preview ...", section "How STQ1_0
 *     works").
 *
 * Block layout (this library's definition; the pages fix only the size):
 *   bytes  0..1   d, IEEE binary16, little-endian
 *   bytes  2..33  4-bit codes: group g (0..63) in byte 2 + 4*(g>>3) + (g&3),
 *                 low nibble when bit 2 of g is clear, high nibble otherwise
 *   bytes 34..41  select bits: group g's bit is bit ((g>>2)&7) of byte
 *                 34 + 4*(g>>5) + (g&3)
 *   code c = nibble | select<<4;  zero lane z = c>>3;  m = c&7; the three
 *   other lanes in increasing order take -1 when their bit of m is set
 *   (lowest lane -> bit 0), else +1.  Decoded weight = +/-fp32(d), or +0.0
 *   in the zero lane.
 * Matrix layout (also this library's): a matrix of n rows and k columns (k a
 * multiple of 256) holds n*k/256 blocks, block b of a row covering columns
 * 256b..256b+255, n*row_bytes(k) bytes in all.  Rows are grouped in tiles of
 * 64 consecutive rows (the last tile holds the n % 64 leftover rows, if any);
 * a tile stores block 0 of each of its rows in row order, then block 1 of
 * each, and so on.  Block b of row r of a matrix starting at byte 0 is at
 *   (t*nb + b*rows_in_tile + (r - t)) * 42,   t = r - r % 64,
 *   rows_in_tile = min(64, n - t),            nb = k / 256.
 * So the 64 rows' block b of a full tile is one contiguous 2688-byte run.
 *
 * Conventions for every entry point:
 *   - array arguments are DEVICE pointers owned by the caller, unless stated;
 *   - work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *     no entry point synchronises the host;
 *   - arguments are validated on the host before any launch; a failed check
 *     returns a status and stq_last_error() holds a message (thread-local);
 *   - STQ_E_HIP means a HIP call (a launch) failed; device faults surface at
 *     the caller's next synchronisation;
 *   - the library allocates no device memory and keeps no device state: the
 *     entry points that need scratch memory (stq_gemv, stq_moe_ffn_decode,
 *     stq_layer_errors) take a caller-owned `workspace` of `workspace_bytes`
 *     bytes, 256-byte aligned, whose required size a host-only query gives
 *     for the same shapes (stq_gemv_plan, stq_moe_ffn_workspace,
 *     stq_layer_errors_workspace); a NULL or smaller workspace is refused
 *     with STQ_E_ARG before any launch.  The workspace is in use until the
 *     call's work on `stream` completes, so calls that run concurrently need
 *     workspaces of their own; its contents between calls are meaningless;
 *   - apart from the thread-local error text the entry points are stateless
 *     and may be called from any number of host threads.
 */
#ifndef STQ_H
#define STQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* stq_stream_t; /* same object as a hipStream_t */

#define STQ_QK 256          /* weights per block */
#define STQ_BLOCK_BYTES 42  /* bytes per block   */

typedef enum {
  STQ_OK = 0,
  STQ_E_ARG = 1,   /* null pointer, bad enum, negative count               */
  STQ_E_SHAPE = 2, /* k not a multiple of 256, sizes inconsistent           */
  STQ_E_ALIGN = 3, /* pointer or stride misaligned                          */
  STQ_E_HIP = 4    /* a HIP runtime call failed                             */
} stq_status;

enum { STQ_ENC_WLS = 0, STQ_ENC_AMAX = 1 };
enum { STQ_X_F32 = 0, STQ_X_BF16 = 1 };

/* Bytes of one packed row of k weights: k/256*42, or -1 if k is not a
 * positive multiple of 256. Pure host function. */
int64_t stq_row_bytes(int64_t k);

/* Encode fp32 rows into STQ1_0 (weighted least squares scale alternating
 * with an importance-weighted choice of the zero lane; lemmy post 66506,
 * paragraph "Scale and zero position are fit together"; amax baseline from
 * the alphasignal.ai summary bullets).
 *   w        [n_rows, k] fp32, row-major, 4-byte aligned, finite values
 *   imatrix  [k] fp32 >= 0, per-column importance; NULL means all ones
 *   encoder  STQ_ENC_WLS: start from the amax pattern (zero the smallest |w|
 *              of each group, signs of w); `rounds` times fit d by weighted
 *              least squares then re-choose every group's zero lane by least
 *              added weighted error q_j*(2|w_j|-d) (lowest lane on ties);
 *              a final fit gives the stored d.
 *            STQ_ENC_AMAX: d = block max |w|, smallest |w| zeroed; `rounds`
 *              ignored.
 *   rounds   >= 0 (3 is the pages' setting)
 *   out      packed matrix, n_rows*k/256*42 bytes (layout above)
 * Sums run in fp64 in a fixed order (lanes of a group in order, then a
 * balanced tree of adjacent groups); d is stored as fp16 via fp32
 * (round-to-nearest-even both times, clamped to 65504).  These rules fix
 * every output byte: any implementation that follows them gives the same
 * bytes.  Non-finite inputs are outside the contract (output unspecified). */
stq_status stq_quantize_rows(const float* w, const float* imatrix, int64_t n_rows, int64_t k,
                             int encoder, int rounds, uint8_t* out, stq_stream_t stream);

/* Decode a packed matrix to fp32: out[r, i] = +/-fp32(d) or +0.0 (bit-exact),
 * the weights the format stands for (every weight of a group is -d, 0 or +d
 * with one zero per group of four, d the block's fp16 scale: lemmy post
 * 66506, paragraph "Four weights, five bits").
 *   q    packed matrix of n_rows rows (layout above), 2-byte aligned
 *   out  [n_rows, k] fp32, row-major */
stq_status stq_dequantize_rows(const uint8_t* q, int64_t n_rows, int64_t k, float* out,
                               stq_stream_t stream);

/* Gathered decode GEMV over (token, expert) pairs, the STQ1_0 matmul of the
 * decode path (lemmy post 66506, paragraph "Runtime": STQ1_0 kernels run the
 * expert projections; each token reaches the top 8 of 256 routed experts,
 * traictory.com "Tencent's 200GB Hy4-preview ...", section "The claim,
 * stated precisely").
 *   w_table   expert e's packed n x k matrix starts at w_table + e*expert_stride_bytes;
 *             w_table 16-byte aligned, expert_stride_bytes a multiple of 16 and
 *             >= n*row_bytes(k)
 *   x         activations [n_tokens, k] with row stride x_row_stride elements,
 *             fp32 (STQ_X_F32, 4-byte aligned) or bf16 bits (STQ_X_BF16,
 *             x_row_stride even, 4-byte aligned rows)
 *   pair_expert, pair_token  int32 [n_pairs]; pair i computes
 *             y[i, :] = W_{pair_expert[i]} x[pair_token[i], :].
 *             NULL pair_expert means expert 0 for every pair; NULL pair_token
 *             means token i for pair i.  Pairs sharing an expert are batched so
 *             the expert's weights stream once per call.  A pair whose expert
 *             is outside [0, n_experts) or whose token is outside
 *             [0, n_tokens) gets a row of NaN.
 *   y         [n_pairs, n] fp32
 *   workspace, workspace_bytes  caller-owned scratch for split outputs, at
 *             least the scratch_bytes stq_gemv_plan reports for these shapes
 *             on this stream's device (may be NULL when that is 0)
 * Accumulation is fp32 with products exact; the summation order is fixed,
 * so repeated calls give identical bits.  The k split, and the parting of an
 * expert with several tokens into up to one k range per token, are chosen
 * per call from the shapes and the CU count of the device `stream` runs on;
 * the environment variable STQ_GEMV_PLAN="s,p" (1 <= s <= k/256 splits,
 * 1 <= p <= 8 parts) replaces that choice, for tuning and tests.  Results
 * meet the same tolerance under every plan; their bits depend on the plan
 * and on the pass form (with bf16 rows and at least as many pairs as
 * experts, a pass of 3 or more tokens runs on the matrix cores), so the same
 * bits on devices of different sizes need the same plan (STQ_GEMV_PLAN). */
stq_status stq_gemv(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts,
                    int64_t n, int64_t k, const void* x, int x_dtype, int64_t x_row_stride,
                    int64_t n_tokens, const int32_t* pair_expert, const int32_t* pair_token,
                    int64_t n_pairs, float* y, void* workspace, int64_t workspace_bytes,
                    stq_stream_t stream);

/* stq_gemv for callers that cannot allocate memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks, plan and results as stq_gemv (bit for
 * bit), without workspace: split outputs go to a fixed scratch array that the
 * library holds on every GPU it runs on, STQ_GEMV_NOALLOC_SCRATCH_BYTES
 * bytes, from the library's load until the process ends.  Shapes whose plan
 * (stq_gemv_plan's scratch_bytes) needs more are refused with STQ_E_SHAPE
 * before any launch.  Every call on one GPU shares that GPU's array, so calls
 * that may run concurrently on one GPU (two streams, two host threads) race
 * and must not overlap; nothing in the array needs to be cleared between
 * calls (every value a call reads was written earlier in the same call).
 * Allocates nothing; the first call on a device looks up that device's copy
 * of the array (STQ_E_HIP if that fails). */
#define STQ_GEMV_NOALLOC_SCRATCH_BYTES (32ll << 20)
stq_status stq_gemv_noalloc(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts,
                            int64_t n, int64_t k, const void* x, int x_dtype, int64_t x_row_stride,
                            int64_t n_tokens, const int32_t* pair_expert, const int32_t* pair_token,
                            int64_t n_pairs, float* y, stq_stream_t stream);

/* The plan stq_gemv takes for these shapes (host only: no GPU work, and no
 * GPU needed when n_cus > 0), so a caller can size its workspace or check a
 * tuning override.  The three outputs are HOST
 * pointers; all must be non-NULL (STQ_E_ARG otherwise).
 *   n_experts, n, k, n_pairs  as for stq_gemv (same checks, same errors)
 *   n_cus        compute units to plan for; 0 = the current device's (256
 *                when no device answers)
 *   splits       out: ranges the k blocks of a row are split into
 *   max_parts    out: most k parts one split is cut into for an expert with
 *                several tokens (an expert with m pairs takes min(m, max_parts))
 *   scratch_bytes  out: workspace bytes the call needs (0 when nothing is split)
 * STQ_GEMV_PLAN is honoured as in stq_gemv.  n_pairs == 0 or n == 0 gives
 * (1, 1, 0): stq_gemv launches nothing then. */
stq_status stq_gemv_plan(int64_t n_experts, int64_t n, int64_t k, int64_t n_pairs, int32_t n_cus,
                         int32_t* splits, int32_t* max_parts, int64_t* scratch_bytes);

/* Routed-expert FFN of one MoE layer for a batch of decode tokens, its
 * expert projections in STQ1_0 (lemmy post 66506, paragraph "Runtime": the
 * routed experts' projections run through STQ1_0 kernels; routing top-k of
 * the routed experts, traictory.com "Tencent's 200GB Hy4-preview ...",
 * section "The claim, stated precisely").  For token t and its pairs
 * p = t*top_k + k, k = 0..top_k-1, with e = pair_expert[p]:
 *     g, u  = rows [0, d_ff) and [d_ff, 2*d_ff) of W_gate_up[e] x_t
 *     h     = silu(g) * u,          silu(v) = v / (1 + exp(-v))   (fp32)
 *     z_p   = W_down[e] h
 *     y[t]  = sum over k, in order, of pair_weight[p] * z_p        (fp32)
 *   w_gate_up  expert e's packed [2*d_ff, d_model] matrix (gate rows, then up
 *              rows) at w_gate_up + e*gate_up_stride_bytes
 *   w_down     expert e's packed [d_model, d_ff] matrix at w_down + e*down_stride_bytes
 *              (both 16-byte aligned, strides multiples of 16 and at least
 *              the packed matrix size; d_model, d_ff multiples of 256)
 *   x          bf16 bits [n_tokens, d_model], row-major
 *   pair_expert int32, pair_weight fp32 [n_tokens*top_k], token-major
 *   y          fp32 [n_tokens, d_model]
 *   workspace, workspace_bytes  caller-owned scratch, at least what
 *              stq_moe_ffn_workspace reports for these shapes on this
 *              stream's device: the pairs' gate/up rows, activations and down
 *              rows (fp32) plus the GEMVs' split outputs
 * Both projections run through the GEMV above (pairs sharing an expert are
 * batched), with h formed once per element between them.  A pair whose
 * expert is outside [0, n_experts) makes its token's row NaN.  At most 65535
 * pairs per call. */
stq_status stq_moe_ffn_decode(const uint8_t* w_gate_up, int64_t gate_up_stride_bytes, const uint8_t* w_down,
                              int64_t down_stride_bytes, int64_t n_experts, int64_t d_model, int64_t d_ff,
                              const uint16_t* x, int64_t n_tokens, const int32_t* pair_expert,
                              const float* pair_weight, int64_t top_k, float* y, void* workspace,
                              int64_t workspace_bytes, stq_stream_t stream);

/* Workspace bytes stq_moe_ffn_decode needs for these shapes on a device with
 * n_cus compute units (0: the current device's); host only, same checks and
 * errors as the call.  workspace_bytes is a HOST pointer; 0 when n_tokens is 0. */
stq_status stq_moe_ffn_workspace(int64_t n_experts, int64_t d_model, int64_t d_ff, int64_t n_tokens,
                                 int64_t top_k, int32_t n_cus, int64_t* workspace_bytes);

/* Grouped GEMM of the prefill path: tokens routed to each expert,
 * grouped by expert, times that expert's STQ1_0 matrix (lemmy post 66506,
 * paragraph "Runtime": STQ1_0 kernels run the routed experts' projections;
 * each token reaches the top 8 of 256 routed experts, traictory.com
 * "Tencent's 200GB Hy4-preview ...", section "The claim, stated precisely",
 * so a prompt's tokens form one dense product per expert).
 *   x_sorted        [total_m, k] bf16 bits, row-major, 16-byte aligned rows
 *                   (k*2 bytes apart)
 *   expert_offsets  DEVICE int32 [n_experts+1], non-decreasing, offsets[0] = 0,
 *                   offsets[n_experts] = total_m: rows offsets[e]..offsets[e+1]-1
 *                   belong to expert e
 *   y               [total_m, n] fp32: y[r, :] = W_e x_sorted[r, :]
 * bf16 x ternary products on matrix cores (exact), fp32 accumulation, one
 * fp32 multiply by d per 256-weight block.  Offsets that break the stated
 * invariants are outside the contract, but the kernel clamps each expert's
 * rows to [0, total_m] (lo = clamp(offsets[e]), hi = clamp(offsets[e+1])
 * and at least lo), so x_sorted and y are never accessed outside their
 * total_m rows: rows in no range are left unwritten and rows in two ranges
 * get either expert's result. */
stq_status stq_grouped_gemm(const uint8_t* w_table, int64_t expert_stride_bytes, int64_t n_experts,
                            int64_t n, int64_t k, const uint16_t* x_sorted,
                            const int32_t* expert_offsets, int64_t total_m, float* y,
                            stq_stream_t stream);

/* Reconstruction error of an approximation W_hat of W under calibration
 * activations, scored with the full Hessian H = X^T X and with its diagonal
 * alone, the two layer-sensitivity measures the pages compare (lemmy post
 * 66506, paragraph "Full-Hessian scoring": off-diagonal terms carry the
 * input correlations that a diagonal-only imatrix misses).  With
 * D = W - W_hat in fp64:
 *     err_full[r] = sum_i (D_r . x_i)^2      = D_r H D_r^T
 *     err_diag[r] = sum_c H_cc D_rc^2,        H_cc = sum_i x_ic^2
 *   w, w_hat   [n_rows, k] fp32, row-major, 16-byte aligned (w_hat is
 *              typically stq_dequantize_rows or stq_q2_roundtrip of w)
 *   x_calib    [n_calib, k] fp32 calibration activations, row-major,
 *              16-byte aligned; n_calib >= 1
 *   err_full, err_diag   [n_rows] fp64, 8-byte aligned
 * Products are exact (fp32 operands in fp64); D X^T accumulates in fp64 on
 * the matrix cores, so the results agree with an fp64 reference to within
 * the fp64 rounding of sums of k and n_calib terms.  The summation order is
 * fixed: repeated calls give identical bits.  Non-finite inputs give
 * non-finite outputs.
 *   workspace, workspace_bytes  caller-owned scratch of at least
 *              stq_layer_errors_workspace bytes: 8*(k + 2*ceil(n_calib/64)*n_rows)
 *              (the diagonal of H, then per-tile partial sums) */
stq_status stq_layer_errors(const float* w, const float* w_hat, int64_t n_rows, int64_t k,
                            const float* x_calib, int64_t n_calib, double* err_full, double* err_diag,
                            void* workspace, int64_t workspace_bytes, stq_stream_t stream);

/* Workspace bytes stq_layer_errors needs (host only; same checks and errors
 * as the call; 0 when n_rows is 0).  workspace_bytes is a HOST pointer. */
stq_status stq_layer_errors_workspace(int64_t n_rows, int64_t k, int64_t n_calib, int64_t* workspace_bytes);

/* Quantize-and-reconstruct through the plain 2-bit format this library uses
 * as the larger partner format of a per-layer allocation (the pages pair
 * STQ1_0 with IQ2_XXS at 2.0625 bits per weight, lemmy post 66506,
 * paragraph "Precision follows weight sensitivity", without defining it; a
 * stand-in of the same size takes its place: 66 bytes per 256 weights).
 * Per 256-weight block: ss = sum of w^2 in fp64 (the four weights of a
 * group in order, then a balanced tree of adjacent groups), s = fp16 of
 * sqrt(ss/256)/2 (fp64 -> fp32 -> fp16, round-to-nearest-even, clamped to
 * 65504); each weight becomes s if |w| < 2s, else 3s, with the sign bit of w.
 *   w, out  [n_rows, k] fp32, row-major, 16-byte aligned (may not overlap)
 * These rules fix every output bit.  Non-finite inputs give unspecified
 * (non-finite) outputs for their block. */
stq_status stq_q2_roundtrip(const float* w, int64_t n_rows, int64_t k, float* out, stq_stream_t stream);

/* Greedy per-byte allocation of the larger format over layers (lemmy post
 * 66506, paragraph "Full-Hessian scoring": layers are taken greedily by
 * error reduction per added byte).  Visit layers by gain/extra_bytes,
 * largest first (lowest index on ties); take a layer when its gain is > 0
 * and the added bytes still fit within `budget`, else skip it.
 *   gain, extra_bytes   HOST double [n_layers]; extra_bytes > 0
 *   chosen              HOST uint8 [n_layers], 1 for a layer taken
 * Pure host function. */
stq_status stq_greedy_allocation(const double* gain, const double* extra_bytes, int64_t n_layers,
                                 double budget, uint8_t* chosen);

/* Measurement helper, not part of the method: reads `bytes` bytes of the
 * device buffer `buf` once with 16-byte loads, the streaming-read rate this
 * GPU sustains, against which the decode GEMV's effective bandwidth is
 * compared (the HBM roofline).  `buf` 16-byte aligned, `bytes` a multiple of
 * 16; `sink` is one device uint32 that may be overwritten (its value is
 * meaningless). */
stq_status stq_stream_read_probe(const void* buf, int64_t bytes, uint32_t* sink, stq_stream_t stream);

/* Measurement helper, not part of the method: the matrix-core reference
 * beside the grouped GEMM's MFMA roofline.  Launches 4096 workgroups of 4
 * wavefronts; each wavefront runs `rounds` rounds of 8 independent
 * v_mfma_f32_16x16x32_bf16 (16,384 flops each) with no memory traffic, so a
 * launch does STQ_MFMA_PROBE_FLOP_PER_ROUND * rounds flops.  `rounds` >= 0
 * (0 launches nothing); `sink` is one device float that is never written in
 * practice (its value is meaningless). */
#define STQ_MFMA_PROBE_FLOP_PER_ROUND 2147483648.0
stq_status stq_mfma_loop_probe(int64_t rounds, float* sink, stq_stream_t stream);

/* Measurement helper, not part of the method: the LDS read rate beside the
 * grouped GEMM's operand reads.  Launches 4096 workgroups of 4 wavefronts;
 * each workgroup fills a 32 KB LDS buffer once, then each wavefront runs
 * `rounds` rounds of 8 LDS reads, each folded into a register (no other
 * memory traffic):
 *   mode 0: ds_read_b128, the 64 lanes reading one contiguous 1 KB run
 *           (conflict free), the form of the GEMM's activation reads;
 *   mode 1: ds_read2_b32 at a per-lane code 0..31 of a 32-entry table and
 *           32 words further (the form of the GEMM's pattern reads).
 * A launch issues STQ_LDS_PROBE_READS_PER_ROUND * rounds wavefront LDS
 * instructions.  `mode` 0 or 1, `rounds` >= 0; `sink` as above (uint32). */
#define STQ_LDS_PROBE_READS_PER_ROUND 131072
stq_status stq_lds_read_probe(int mode, int64_t rounds, uint32_t* sink, stq_stream_t stream);

/* Static text of a status code. */
const char* stq_status_string(stq_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* stq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STQ_H */
