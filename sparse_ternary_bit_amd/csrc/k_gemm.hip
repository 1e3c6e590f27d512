// Grouped GEMM of the prefill path: for every expert e, the tokens routed to
// it (rows offsets[e] .. offsets[e+1]-1 of x_sorted, bf16) times the expert's
// STQ1_0 matrix, y[r, :] = W_e x_sorted[r, :], fp32 out.
//
// The pages say only that STQ1_0 runs through dedicated GPU kernels
// (lemmy.durstig.online post 66506, "Runtime"); a prefill batch makes this a
// real dense contraction, so it runs on the bf16 matrix cores of gfx950
// (v_mfma_f32_16x16x32_bf16).  Ternary weights are exact in bf16 and a bf16 x
// bf16 product is exact in fp32; sums are fp32, and each 256-weight block's
// partial sum is scaled by its fp32(d) once (one FMA per output per block).
//
// Work unit: a workgroup of 4 wavefronts owns 256 weight rows (one 64-row
// tile of the packed matrix per wavefront) of one expert and all of that
// expert's tokens, in passes of at most 80 tokens (5 tiles of 16).  Every
// weight is therefore decoded once per pass, and each decoded MFMA operand
// is reused for every token tile of the pass.  Two workgroups share a CU
// (about 69 KB of LDS and 256 VGPRs per wavefront each), so the barriers and
// block boundaries of one overlap the other's matrix-core work.
//
// Per 256-weight block b:
//   * activations stream from global memory straight into LDS (16-byte
//     direct loads) half a block (128 per token) at a time into the second
//     of two buffers while the other half is multiplied; a token's 16
//     16-byte chunks of a half are stored XOR-swizzled by the token index
//     (mod 16) so the matrix-operand reads below are bank-conflict free;
//   * each wavefront's contiguous tile run of block b+1 streams into LDS the
//     same way; each lane then reads its own row's 42-byte block there,
//     realigns it and turns it into four 16-byte records, one per MFMA
//     k-quarter: for each of the block's 8 k-steps the quarter's two group
//     codes, pre-scaled by 4 so a code is directly a byte offset into the
//     pattern table;
//   * per half block an MFMA lane reads its four row tiles' record words for
//     the half's 4 k-steps (two 16-byte reads), and per k-step and row tile
//     extracts two codes (two bit-field extracts) and reads the bf16 lanes
//     of both patterns from a 32-entry table in LDS (two 8-byte reads): that
//     is the whole weight decode.  The k-steps are software-pipelined: step
//     s+1's operand reads are issued before step s's MFMAs;
//   * after the block's 8 k-steps the fp32 partial sums are scaled by the
//     rows' d into the fp32 totals.
// Two barriers per block (one per half).  Workgroups of one expert are
// launched on the same XCD (workgroup ids are dealt to the 8 XCDs round
// robin), so the expert's activations are fetched once into that XCD's L2
// and shared by its 16 slabs.
#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSlab = kWaves * kTileRows;   // 256 weight rows per workgroup
constexpr int kMaxTiles = 5;                // token tiles of 16 per pass
constexpr int kMaxTok = kMaxTiles * 16;     // 80 tokens per pass
constexpr int kHalfBytes = kQK;             // one token's 128 activations: half a block
constexpr int kXBuf = kMaxTok * kHalfBytes; // 20480 bytes per buffer
constexpr int kXcds = 8;
constexpr int kWRaw = 3 * 1024;             // 16-byte aligned window over one 2688-byte tile run

struct GArgs {
  const uint8_t* w;
  int64_t estride;
  int n_experts;
  int n;
  int nb;
  int64_t k;
  const uint16_t* x;
  const int32_t* offsets;
  int64_t total_m;
  float* y;
  int nslab;
  int vec4;  // n % 4 == 0: outputs stored 16 bytes at a time
};

struct Smem {
  // Pattern table: entry c of lut[0..31] holds lanes 0,1 of code c as bf16,
  // entry c of lut[32..63] lanes 2,3.  Kept at byte 0 so a code times 4 is
  // its address.
  uint32_t lut[64];
  float dsc[kWaves][kTileRows];           // fp32(d) of each row's current block
  // records: word s2 (k-steps 2*s2, 2*s2+1) of quarter q of row r of row tile
  // i sits at rec[wave][s2][q][r][i], so an MFMA lane's four row-tile words
  // are one 16-byte read and a wavefront reads 1 KB in one contiguous run
  // (the writers, a row tile per 16 lanes, meet 2-way bank conflicts on
  // their 4-byte stores, which cost less than the 4-byte reads they replace)
  alignas(16) uint32_t rec[kWaves][4][4][16][4];
  alignas(16) char x[2][kXBuf];           // activations, current and next half block
  alignas(16) char wraw[kWaves][kWRaw];   // each wavefront's tile run of the next block
};

// A zero the compiler cannot see through: the first MFMA of each block adds
// to these registers instead of to freshly zeroed accumulators.
__device__ __forceinline__ float opaque_zero() {
  float z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// A pass: tokens [row0, row0 + mt) of the sorted activations, NT = ceil(mt/16).
// The thread index through an opaque move: values derived from it are then
// computed in each pass instead of being hoisted to the kernel's start, where
// the register pressure of the passes would spill them to scratch memory.
__device__ __forceinline__ int pass_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(static_cast<int>(threadIdx.x)));
  return t;
}

template <int NT>
__device__ __forceinline__ void run_pass(const GArgs& a, Smem& sh, const uint8_t* wexp, int slab, int64_t row0,
                                         int mt) {
  const int tid = pass_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r = lane & 15;

  // this wavefront's weight rows: one 64-row tile of the packed matrix
  const int trow0 = slab * kSlab + wave * kTileRows;
  const int valid = max(0, min(kTileRows, a.n - trow0));
  const uint8_t* tb = wexp + static_cast<int64_t>(min(trow0, a.n)) * a.nb * kBlockBytes;
  const Rsrc rs = make_rsrc(tb, (static_cast<uint32_t>(valid) * a.nb * kBlockBytes + 3u) & ~3u);

  // activations, half a block (128 of them, 16 chunks of 16 bytes) per token
  // at a time: 4 tokens per wavefront instruction; chunk c of token t goes to
  // slot c ^ (t & 15) of the token's 256 bytes.  Wavefront w stages
  // instructions j = w, w + 4, ...: this lane's token t = 4j + lane / 16 moves
  // by 16 tokens per step and t & 15, so the chunk c, stays the same; tokens
  // past the pass (t >= mt) read zeros through the range check and are not
  // stored
  const int n_ins = (mt + 3) >> 2;
  const uint32_t xrow = static_cast<uint32_t>(a.k) * 2;
  const Rsrc xs_rs = make_rsrc(a.x + row0 * a.k, static_cast<uint32_t>(mt) * xrow);
  const int t_first = 4 * wave + (lane >> 4);
  const uint32_t x_first = static_cast<uint32_t>(t_first) * xrow + (((lane & 15) ^ (t_first & 15)) * 16);
  auto stage_x = [&](int h, int buf) {
    uint32_t voff = x_first + static_cast<uint32_t>(h) * kHalfBytes;
    for (int j = wave; j < n_ins; j += kWaves, voff += 16 * xrow)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xs_rs, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(sh.x[buf] + j * 1024)),
          16, static_cast<int>(voff), 0, 0, 0);
  };

  // the tile run of block b (valid * 42 bytes) into this wavefront's window,
  // from the 16-byte boundary at or below its start; the buffer range check
  // turns bytes past the tile into zeros
  auto run_start = [&](int b) { return static_cast<uint32_t>(b) * valid * kBlockBytes; };
  auto stage_w = [&](int b) {
    const uint32_t st = run_start(b) & ~15u;
#pragma unroll
    for (int j = 0; j < kWRaw / 1024; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(sh.wraw[wave] + j * 1024)),
          16, static_cast<int>(st + j * 1024 + lane * 16), 0, 0, 0);
  };
  // this lane's block out of the window: the 11 aligned words around it
  auto block_from_window = [&](int b) {
    const uint32_t off = (run_start(b) & 15u) + lane * kBlockBytes;
    const uint32_t* wv = reinterpret_cast<const uint32_t*>(sh.wraw[wave] + (off & ~3u));
    RawBlock rw;
#pragma unroll
    for (int i = 0; i < 11; ++i) rw.w[i] = wv[i];
    return realign_block(rw, (off & 2u) != 0);
  };

  // records of one block from this lane's own row
  auto make_records = [&](const Block& blk) {
    uint32_t cl[8], cu[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t W = blk.qs[s];
      const uint32_t QH = blk.qh[s >> 2];
      const int sh6 = 6 - 2 * (s & 3);
      // byte j of cl: 4 * code of group 8s+j; of cu: 4 * code of group 8s+4+j
      cl[s] = ((W << 2) & 0x3C3C3C3Cu) | ((QH << sh6) & 0x40404040u);
      cu[s] = ((W >> 2) & 0x3C3C3C3Cu) | (((QH >> 1) << sh6) & 0x40404040u);
    }
    // quarter q covers groups 8s+2q, 8s+2q+1 of k-step s: bytes (2q, 2q+1) of
    // cl for q < 2, of cu for q >= 2
    const int ti = lane >> 4, tr = lane & 15;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      sh.rec[wave][s2][0][tr][ti] = __builtin_amdgcn_perm(cl[2 * s2 + 1], cl[2 * s2], 0x05040100u);
      sh.rec[wave][s2][1][tr][ti] = __builtin_amdgcn_perm(cl[2 * s2 + 1], cl[2 * s2], 0x07060302u);
      sh.rec[wave][s2][2][tr][ti] = __builtin_amdgcn_perm(cu[2 * s2 + 1], cu[2 * s2], 0x05040100u);
      sh.rec[wave][s2][3][tr][ti] = __builtin_amdgcn_perm(cu[2 * s2 + 1], cu[2 * s2], 0x07060302u);
    }
    sh.dsc[wave][lane] = half_bits_to_float(blk.d16);
  };


  // B operand addresses: token 16*bt + r, chunk 4s + q of its half block
  // (s the k-step within the half) in slot (4s + q) ^ r = (4s) ^ q ^ r
  const int u = q ^ r;
  int xb[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) xb[s4] = r * kHalfBytes + ((4 * s4) ^ u) * 16;

  const f32x4_t zero4 = {opaque_zero(), opaque_zero(), opaque_zero(), opaque_zero()};
  f32x4_t tot[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) tot[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: block 0 (its first half of activations, its weights)
  stage_x(0, 0);
  stage_w(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads have landed
  make_records(block_from_window(0));
  __syncthreads();

  // operands of k-step s: A[i] (row tile i) from the two group codes of the
  // record word for this k-step pair, B[t] (token tile t) from the activations
  auto decode_a = [&](const u32x4_t& Rw, int s, bf16x8_t (&A)[4]) {
    const char* lut = reinterpret_cast<const char*>(sh.lut);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = Rw[i];
      const uint32_t c1 = __builtin_amdgcn_ubfe(w, 16 * (s & 1), 8);
      const uint32_t c2 = __builtin_amdgcn_ubfe(w, 16 * (s & 1) + 8, 8);
      u32x4_t v;
      v[0] = *reinterpret_cast<const uint32_t*>(lut + c1);
      v[1] = *reinterpret_cast<const uint32_t*>(lut + c1 + 128);
      v[2] = *reinterpret_cast<const uint32_t*>(lut + c2);
      v[3] = *reinterpret_cast<const uint32_t*>(lut + c2 + 128);
      A[i] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  auto read_b = [&](const char* xs, int s, bf16x8_t (&B)[NT]) {
    const int xo = xb[s & 3];
#pragma unroll
    for (int t = 0; t < NT; ++t) B[t] = *reinterpret_cast<const bf16x8_t*>(xs + xo + t * 16 * kHalfBytes);
  };

  for (int b = 0; b < a.nb; ++b) {
    const bool more = b + 1 < a.nb;
    // The block's four record words (one per k-step pair) and, per half
    // block, a software pipeline over its 4 k-steps: the operands of step
    // s + 1 are read from LDS before the MFMAs of step s are issued.
    bf16x8_t A[2][4], Bv[2][NT];
    f32x4_t part[4][NT];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int h = 2 * b + half;
      const int buf = h & 1;
      // the next half block's activations (and, in the first half, the next
      // block's weights) stream into LDS while this half is multiplied
      if (half == 0 || more) stage_x(h + 1, buf ^ 1);
      if (half == 0 && more) stage_w(b + 1);
      const char* xs = sh.x[buf];
      // this half's two record words (k-step pairs 2 half, 2 half + 1)
      u32x4_t R[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        R[s2] = *reinterpret_cast<const u32x4_t*>(&sh.rec[wave][2 * half + s2][q][r][0]);
      decode_a(R[0], 4 * half, A[0]);
      read_b(xs, 0, Bv[0]);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int s = 4 * half + sl;
        const int cur = sl & 1;
        if (sl + 1 < 4) {
          decode_a(R[(sl + 1) >> 1], s + 1, A[cur ^ 1]);
          read_b(xs, sl + 1, Bv[cur ^ 1]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4_t c = (s == 0) ? zero4 : part[i][t];
            part[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[cur][i], Bv[cur][t], c, 0, 0, 0);
          }
        }
        // keep each step's reads (for the next step) and MFMAs together
        __builtin_amdgcn_sched_barrier(0);
      }
      if (half == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of the second half is in LDS
      } else {
        // scale the block's partial sums: rows 16i + 4q + j of the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sh.dsc[wave][16 * i + 4 * q]);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) tot[i][t][j] = fmaf(d4[j], part[i][t][j], tot[i][t][j]);
        }
        if (more) {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // block b+1's weights and first activations are in LDS
          make_records(block_from_window(b + 1));
        }
      }
      __syncthreads();
    }
  }

  // y[row0 + 16t + r, trow0 + 16i + 4q + j]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = 16 * t + r;
    if (tok >= mt) continue;
    float* yr = a.y + (row0 + tok) * a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = trow0 + 16 * i + 4 * q;
      if (a.vec4 && col + 3 < a.n) {
        *reinterpret_cast<f32x4_t*>(yr + col) = tot[i][t];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col + j < a.n) yr[col + j] = tot[i][t][j];
      }
    }
  }
}

// Two workgroups per CU (LDS ~69 KB each, 256 VGPRs per wavefront), so one
// workgroup's barriers and block boundaries overlap the other's MFMAs.
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(GArgs a) {
  __shared__ Smem sh;
  // workgroup -> (expert, slab): the slabs of one expert share an XCD
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int local = wg / kXcds;
  const int slab = local % a.nslab;
  const int e = (local / a.nslab) * kXcds + xcd;
  if (e >= a.n_experts) return;
  // the expert's rows, clamped to [0, total_m] so that offsets outside the
  // contract can neither read past x_sorted nor write past y
  const int64_t lo = min(max(static_cast<int64_t>(a.offsets[e]), int64_t{0}), a.total_m);
  const int64_t hi = min(max(static_cast<int64_t>(a.offsets[e + 1]), lo), a.total_m);
  const int m0 = static_cast<int>(lo);
  const int m = static_cast<int>(hi - lo);
  if (m <= 0) return;

  if (threadIdx.x < 32) {
    const uint32_t c = threadIdx.x;
    auto bf = [&](int lane) -> uint32_t {
      const int t = code_lane_value(c, lane);
      return t == 0 ? 0u : (t > 0 ? 0x3F80u : 0xBF80u);  // bf16 +1, -1
    };
    sh.lut[c] = bf(0) | (bf(1) << 16);
    sh.lut[32 + c] = bf(2) | (bf(3) << 16);
  }
  __syncthreads();

  const uint8_t* wexp = a.w + static_cast<int64_t>(e) * a.estride;
  const int np = (m + kMaxTok - 1) / kMaxTok;
  const int per = (m + np - 1) / np;
  for (int p = 0; p < np; ++p) {
    const int base = p * per;
    const int mt = min(per, m - base);
    const int64_t row0 = static_cast<int64_t>(m0) + base;
    switch ((mt + 15) >> 4) {
      case 1: run_pass<1>(a, sh, wexp, slab, row0, mt); break;
      case 2: run_pass<2>(a, sh, wexp, slab, row0, mt); break;
      case 3: run_pass<3>(a, sh, wexp, slab, row0, mt); break;
      case 4: run_pass<4>(a, sh, wexp, slab, row0, mt); break;
      default: run_pass<5>(a, sh, wexp, slab, row0, mt); break;
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& ga, hipStream_t s) {
  if (ga.total_m == 0 || ga.n == 0 || ga.n_experts == 0) return hipSuccess;
  GArgs a{};
  a.w = ga.w_table;
  a.estride = ga.expert_stride;
  a.n_experts = static_cast<int>(ga.n_experts);
  a.n = static_cast<int>(ga.n);
  a.nb = static_cast<int>(ga.k / kQK);
  a.k = ga.k;
  a.x = ga.x;
  a.offsets = ga.offsets;
  a.total_m = ga.total_m;
  a.y = ga.y;
  a.nslab = static_cast<int>((ga.n + kSlab - 1) / kSlab);
  a.vec4 = (ga.n % 4) == 0;
  const int64_t groups = (ga.n_experts + kXcds - 1) / kXcds;
  const int64_t grid = groups * kXcds * a.nslab;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace stq
