// Gathered STQ1_0 GEMV for the decode path: y[pair, :] = W_expert x_token.
//
// The pages say only that STQ1_0 runs through dedicated GPU kernels at about
// the speed of IQ1_M (lemmy.durstig.online post 66506, "Runtime"); the design
// below is this library's, for gfx950.
//
// Work unit: a workgroup of 512 threads owns 512 consecutive rows of one
// expert (one row per thread, eight 64-row tiles) and a range of 256-weight
// blocks along k, for up to kMT tokens at a time.  The (token, expert) pair
// list is scanned on the device: the first valid pair of an expert leads and
// collects every later pair with that expert, so the expert's weights stream
// once per kMT tokens.
//
// Inner product per block: a group of four weights holds one of 32 patterns,
// so for each token and group the 32 possible signed sums of its four
// activations are tabulated in LDS once per workgroup (512 rows share each
// table).  A row then costs, per group, one bit-field extract of its 5-bit
// code (already scaled by 4) and, per token, one LDS read with the group's
// table offset as an immediate plus one fp32 add; the block's fp16 scale
// multiplies the block sum.  All threads of a wavefront read the same group's
// 128-byte table at once, so the reads are bank-conflict free.  Tables are
// double-buffered: while block b is summed from one buffer, block b+1's table
// is built into the other, one barrier per block.
//
// Weights: the matrix is stored in 64-row tiles, block-major inside a tile,
// so a wavefront's 64 rows of block b are one contiguous 2688-byte run.  Each
// thread loads the 11 aligned words that cover its own 42-byte block with
// 16 + 16 + 12-byte buffer loads (the wavefront's loads cover the run with no
// gaps and never leave it) and realigns them with byte permutes.  Loads run
// two blocks ahead, in the order they are consumed.
//
// k split: the blocks of a row may be split over several workgroups (chosen
// per call from the expected number of active experts, see plan_gemv); each
// writes fp32 partial sums to scratch and a second small kernel adds them in
// split order, so the result does not depend on scheduling.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

constexpr int kRows = 512;                 // rows (= threads) per workgroup
constexpr int kWaves = kRows / 64;
constexpr int kMT = 4;                     // tokens per pass
constexpr int kTabBytes = kGroups * 32 * 4;
constexpr int kTokStride = kTabBytes + 16; // token tables apart by a non-multiple of 256 bytes
constexpr int kBufBytes = kMT * kTokStride;

struct KArgs {
  const uint8_t* w;
  int64_t estride;
  int n_experts;
  int n;
  int nb;          // blocks per row
  const void* x;
  int64_t xstride;
  int n_tokens;
  const int32_t* pe;
  const int32_t* pt;
  int n_pairs;
  float* y;
  int bps;         // blocks per split
  int splits;
  float* partial;  // [splits, n_pairs, n] when splits > 1
  int ppt;         // without pair_token: pair q uses token q / ppt
  int64_t ff;      // SwiGLU activations: offset of the "up" half in a row
};

__device__ __forceinline__ int pair_expert(const KArgs& a, int q) { return a.pe ? a.pe[q] : 0; }
__device__ __forceinline__ int pair_token(const KArgs& a, int q) { return a.pt ? a.pt[q] : q / a.ppt; }

struct Shared {
  alignas(16) char tab[2][kBufBytes];       // two table buffers; per token 32 signed sums x 64 groups
  int pairs[kMT];
  int toks[kMT];
  int mc;
  int next;
  int lead;
  int flag;
  unsigned long long ball[kWaves];
};

// Collect up to kMT pairs with expert e and a valid token, from `cursor` on,
// in index order.  Leaves the count in sh.mc and the resume index in sh.next.
__device__ void gather(const KArgs& a, Shared& sh, int e, int cursor) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    sh.mc = 0;
    sh.next = a.n_pairs;
  }
  __syncthreads();
  for (int base = cursor; base < a.n_pairs; base += kRows) {
    const int q = base + tid;
    bool match = false;
    if (q < a.n_pairs) {
      const int tq = pair_token(a, q);
      match = pair_expert(a, q) == e && tq >= 0 && tq < a.n_tokens;
    }
    const unsigned long long bal = __ballot(match);
    if (lane == 0) sh.ball[wave] = bal;
    __syncthreads();
    if (tid == 0) {
      int mc = sh.mc;
      int next = base + kRows;
      for (int w = 0; w < kWaves && mc < kMT; ++w) {
        unsigned long long bm = sh.ball[w];
        while (bm != 0ull && mc < kMT) {
          const int bit = __ffsll(static_cast<long long>(bm)) - 1;
          bm &= bm - 1ull;
          const int qq = base + 64 * w + bit;
          sh.pairs[mc] = qq;
          sh.toks[mc] = pair_token(a, qq);
          ++mc;
          next = qq + 1;
        }
      }
      if (mc < kMT) next = base + kRows;
      sh.mc = mc;
      sh.next = next;
    }
    __syncthreads();
    if (sh.mc >= kMT) break;
  }
}

// Activations of one group (4 values) of one token at column `col`, by
// source kind: fp32 rows, bf16 rows, or SwiGLU of fp32 gate/up rows
// (value = silu(row[col]) * row[ff + col], silu(v) = v / (1 + exp(-v))).
enum XMode { kXF32 = 0, kXBF16 = 1, kXSwiGLU = 2 };

template <int kMode>
struct XGroup {
  static constexpr int kWords = kMode == kXBF16 ? 2 : (kMode == kXSwiGLU ? 8 : 4);
  uint32_t v[kWords];
  __device__ __forceinline__ void load(const KArgs& a, int tok, int64_t col) {
    if constexpr (kMode == kXBF16) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) + tok * a.xstride + col);
      v[0] = p[0];
      v[1] = p[1];
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.x) + tok * a.xstride + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = p[i];
      if constexpr (kMode == kXSwiGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 + i] = p[a.ff + i];
      }
    }
  }
  __device__ __forceinline__ float get(int j) const {
    if constexpr (kMode == kXBF16) {
      return __uint_as_float(j & 1 ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16));
    } else if constexpr (kMode == kXSwiGLU) {
      const float g = __uint_as_float(v[j]);
      return g / (1.0f + expf(-g)) * __uint_as_float(v[4 + j]);
    } else {
      return __uint_as_float(v[j]);
    }
  }
};

// Table entries 8z..8z+7 of one group for zero lane z.  Entry 8z+m is the sum
// over the three kept lanes (in order) of -x or +x as bit r of m says.
template <int kMode>
__device__ __forceinline__ void build_entries(const XGroup<kMode>& xg, int z, char* dst) {
  const float x0 = xg.get(0), x1 = xg.get(1), x2 = xg.get(2), x3 = xg.get(3);
  const float a = (z == 0) ? x1 : x0;
  const float b = (z <= 1) ? x2 : x1;
  const float c = (z <= 2) ? x3 : x2;
  const float u0 = a + b;   // +a +b
  const float u1 = b - a;   // -a +b
  const float e0 = u0 + c, e1 = u1 + c, e2 = c - u1, e3 = c - u0;
  float4* o = reinterpret_cast<float4*>(dst);
  o[0] = make_float4(e0, e1, e2, e3);
  o[1] = make_float4(-e3, -e2, -e1, -e0);
}

// Sum over the 64 groups of one block of table[code], for MC tokens.
template <int MC>
__device__ __forceinline__ void block_dot(const char* tab, const Block& blk, float (&acc)[kMT]) {
  const float d = half_bits_to_float(blk.d16);
  float bs[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) bs[m] = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t Q = blk.qs[w];
    const uint32_t Hs = blk.qh[w >> 2] << (6 - 2 * (w & 3));
    // byte j of cl / cu = 4 * code of group 8w+j / 8w+4+j
    uint32_t cl = ((Q << 2) & 0x3C3C3C3Cu) | (Hs & 0x40404040u);
    uint32_t cu = ((Q >> 2) & 0x3C3C3C3Cu) | ((Hs >> 1) & 0x40404040u);
    // Opaque to the optimiser: knowing bits 0, 1 and 7 of every byte are
    // zero, it would shrink a byte extract's mask to 0x7C and emit a shift
    // and an AND; hidden, each extract below is one v_bfe_u32.
    asm("" : "+v"(cl), "+v"(cu));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ol = __builtin_amdgcn_ubfe(cl, 8 * j, 8);
      const uint32_t ou = __builtin_amdgcn_ubfe(cu, 8 * j, 8);
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        bs[m] += *reinterpret_cast<const float*>(tab + ol + (m * kTokStride + (8 * w + j) * 128));
        bs[m] += *reinterpret_cast<const float*>(tab + ou + (m * kTokStride + (8 * w + 4 + j) * 128));
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = fmaf(d, bs[m], acc[m]);
}

// Process blocks [b_begin, b_end) of this workgroup's rows for MC tokens.
template <int kMode, int MC>
__device__ __forceinline__ void run_chunk(const KArgs& a, Shared& sh, const uint8_t* wexp, int b_begin,
                                          int b_end, float (&acc)[kMT]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // table items of this thread: item i = 256*m + 4*g + z, items tid and tid + 512
  constexpr int kItems = 256 * MC;
  const int it_g = (tid >> 2) & 63, it_z = tid & 3;
  const int m0 = tid >> 8, m1 = m0 + 2;
  const bool has0 = tid < kItems, has1 = tid + kRows < kItems;
  int tok[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) tok[m] = __builtin_amdgcn_readfirstlane(sh.toks[m]);
  int tok0 = 0, tok1 = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    if (m == m0) tok0 = tok[m];
    if (m == m1) tok1 = tok[m];
  }
  const int tab_off0 = m0 * kTokStride + it_g * 128 + it_z * 32;
  const int tab_off1 = m1 * kTokStride + it_g * 128 + it_z * 32;

#pragma unroll
  for (int m = 0; m < kMT; ++m) acc[m] = 0.0f;

  // this wavefront's rows are one tile of the packed matrix
  const int rowbase = blockIdx.x * kRows + wave * 64;
  const int valid = max(0, min(kTileRows, a.n - rowbase));
  const uint8_t* tb = wexp + static_cast<int64_t>(min(rowbase, a.n)) * a.nb * kBlockBytes;
  const Rsrc rs = make_rsrc(tb, (static_cast<uint32_t>(valid) * a.nb * kBlockBytes + 3u) & ~3u);
  auto load_w = [&](RawBlock& r, int b) {
    load_raw_block(rs, (static_cast<uint32_t>(b) * valid + lane) * kBlockBytes, r);
  };
  auto load_x = [&](XGroup<kMode> (&x)[2], int b) {
    const int64_t col = static_cast<int64_t>(b) * kQK + 4 * it_g;
    if (has0) x[0].load(a, tok0, col);
    if (has1) x[1].load(a, tok1, col);
  };
  auto build = [&](const XGroup<kMode> (&x)[2], char* t) {
    if (has0) build_entries<kMode>(x[0], it_z, t + tab_off0);
    if (has1) build_entries<kMode>(x[1], it_z, t + tab_off1);
  };
  // 42*(b*valid + lane) is 2 mod 4 exactly when b*valid + lane is odd
  const bool lane_odd = (lane & 1) != 0;
  char* buf0 = sh.tab[0];
  char* buf1 = sh.tab[1];

  // Pipeline over blocks j = b - b_begin: weights of blocks j, j+1 and
  // activations of blocks j+1, j+2 are in flight; block j uses weight slot
  // j&1, table buffer j&1, and builds table j+1 from activation slot (j+1)&1.
  RawBlock wa, wb;
  XGroup<kMode> xa[2], xb[2];
  auto step = [&](RawBlock& wcur, XGroup<kMode> (&xnext)[2], char* tcur, char* tnext, int b) {
    const bool odd = ((static_cast<uint32_t>(b) * valid) & 1u) ? !lane_odd : lane_odd;
    const Block blk = realign_block(wcur, odd);
    if (b + 1 < b_end) build(xnext, tnext);
    if (b + 2 < b_end) load_w(wcur, b + 2);
    if (b + 3 < b_end) load_x(xnext, b + 3);
    block_dot<MC>(tcur, blk, acc);
    __syncthreads();  // table b+1 is complete and every thread is done with table b
  };
  {
    load_w(wa, b_begin);
    if (b_begin + 1 < b_end) load_w(wb, b_begin + 1);
    XGroup<kMode> x0[2];
    load_x(x0, b_begin);
    if (b_begin + 1 < b_end) load_x(xb, b_begin + 1);
    if (b_begin + 2 < b_end) load_x(xa, b_begin + 2);
    build(x0, buf0);
    __syncthreads();
  }
  for (int b = b_begin; b < b_end; b += 2) {
    step(wa, xb, buf0, buf1, b);
    if (b + 1 < b_end) step(wb, xa, buf1, buf0, b + 1);
  }
}

// A pair leads when its token is valid and no earlier valid pair names the
// same expert; the leading pair of an expert collects all of that expert's
// pairs (gather above).  Workgroup z serves the z-th leading pair in pair
// order, so the workgroups with work are the first ones launched whatever
// the order of the pairs: workgroups are dealt to the shader engines of an
// XCD round robin, and a periodic pattern of idle workgroups (pairs sorted by
// expert, say, with four pairs per expert) would otherwise put all the work
// on one of them.
constexpr int kLeadExperts = static_cast<int>(sizeof(Shared::tab) / sizeof(int));

__device__ __forceinline__ bool pair_valid(const KArgs& a, int q, int& e) {
  e = pair_expert(a, q);
  const int t = pair_token(a, q);
  return e >= 0 && e < a.n_experts && t >= 0 && t < a.n_tokens;
}

// With at most kLeadExperts experts: the first valid pair of every expert by
// an LDS atomic minimum (in the table space, unused until the tables are
// built), then a running count of leading pairs in pair order until the z-th.
__device__ int find_leader(const KArgs& a, Shared& sh, int z) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* first = reinterpret_cast<int*>(&sh.tab[0][0]);
  for (int e = tid; e < a.n_experts; e += kRows) first[e] = 0x7FFFFFFF;
  if (tid == 0) sh.lead = -1;
  __syncthreads();
  for (int q = tid; q < a.n_pairs; q += kRows) {
    int e;
    if (pair_valid(a, q, e)) atomicMin(&first[e], q);
  }
  __syncthreads();
  int base = 0;
  for (int c = 0; c < a.n_pairs && base <= z; c += kRows) {
    const int q = c + tid;
    int e = -1;
    const bool lead = q < a.n_pairs && pair_valid(a, q, e) && first[e] == q;
    const unsigned long long bal = __ballot(lead);
    if (lane == 0) sh.ball[wave] = bal;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cw = __popcll(sh.ball[w]);
      before += (w < wave) ? cw : 0;
      total += cw;
    }
    const int rank = base + before + __popcll(bal & ((1ull << lane) - 1ull));
    if (lead && rank == z) sh.lead = q;
    base += total;
    __syncthreads();  // sh.ball is rewritten by the next chunk
  }
  return sh.lead;  // sh.lead is not written again in this launch
}

// Beyond kLeadExperts experts: workgroup z serves pair z if it leads (a scan
// of the earlier pairs), so idle workgroups are interleaved with busy ones.
__device__ int leader_if_first(const KArgs& a, Shared& sh, int z) {
  const int tid = threadIdx.x;
  int e;
  if (!pair_valid(a, z, e)) return -1;
  e = __builtin_amdgcn_readfirstlane(e);
  if (tid == 0) sh.flag = 0;
  __syncthreads();
  for (int q = tid; q < z; q += kRows) {
    int eq;
    if (pair_valid(a, q, eq) && eq == e) sh.flag = 1;
  }
  __syncthreads();
  return sh.flag ? -1 : z;
}

template <int kMode>
__device__ __forceinline__ void gemv_main(const KArgs& a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int z = blockIdx.z;
  const int split = blockIdx.y;
  const int row = blockIdx.x * kRows + tid;
  const bool row_ok = row < a.n;

  // an invalid pair z gets a row of NaN, whichever workgroup leads below
  {
    const int ez = pair_expert(a, z), tz = pair_token(a, z);
    if ((ez < 0 || ez >= a.n_experts || tz < 0 || tz >= a.n_tokens) && split == 0 && row_ok)
      a.y[static_cast<int64_t>(z) * a.n + row] = __builtin_nanf("");
  }
  // this workgroup leads the z-th leading pair (uniform; -1 if there are fewer)
  const int p = __builtin_amdgcn_readfirstlane(a.n_experts <= kLeadExperts ? find_leader(a, sh, z)
                                                                             : leader_if_first(a, sh, z));
  if (p < 0) return;
  const int e = __builtin_amdgcn_readfirstlane(pair_expert(a, p));

  const uint8_t* wexp = a.w + static_cast<int64_t>(e) * a.estride;
  const int b_begin = split * a.bps;
  const int b_end = min(a.nb, b_begin + a.bps);

  int cursor = p;
  for (;;) {
    gather(a, sh, e, cursor);
    const int mc = __builtin_amdgcn_readfirstlane(sh.mc);
    if (mc == 0) break;
    cursor = __builtin_amdgcn_readfirstlane(sh.next);
    float acc[kMT];
    switch (mc) {
      case 1: run_chunk<kMode, 1>(a, sh, wexp, b_begin, b_end, acc); break;
      case 2: run_chunk<kMode, 2>(a, sh, wexp, b_begin, b_end, acc); break;
      case 3: run_chunk<kMode, 3>(a, sh, wexp, b_begin, b_end, acc); break;
      default: run_chunk<kMode, 4>(a, sh, wexp, b_begin, b_end, acc); break;
    }
    if (row_ok) {
#pragma unroll
      for (int m = 0; m < kMT; ++m) {
        if (m < mc) {
          const int64_t q = sh.pairs[m];
          if (a.splits == 1) a.y[q * a.n + row] = acc[m];
          else a.partial[(static_cast<int64_t>(split) * a.n_pairs + q) * a.n + row] = acc[m];
        }
      }
    }
    __syncthreads();  // sh.pairs is rewritten by the next gather
  }
}

template <int kMode>
__global__ __launch_bounds__(kRows) void gemv_kernel(KArgs a) {
  gemv_main<kMode>(a);
}

// SwiGLU rows (the FFN's down projection) build their tables through an
// exponential and need more registers; held to 128 VGPRs, two workgroups
// still fit per CU (unbounded they take 139 and one).  The bf16 and fp32
// variants fit without the bound and run faster without it.
__global__ __launch_bounds__(kRows, 4) void gemv_kernel_swiglu(KArgs a) {
  gemv_main<kXSwiGLU>(a);
}

// y[p, r] = sum over splits s, in order, of partial[s, p, r], for valid pairs.
// The loads of 16 splits are issued before their adds, so the loop pays one
// memory latency per 16 splits; the additions stay in split order.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ partial, int splits,
                                                            int64_t plane, const int32_t* __restrict__ pe,
                                                            const int32_t* __restrict__ pt, int ppt, int n_experts,
                                                            int n_tokens, int n, float* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= plane) return;
  const int p = static_cast<int>(i / n);
  const int e = pe ? pe[p] : 0;
  const int t = pt ? pt[p] : p / ppt;
  if (e < 0 || e >= n_experts || t < 0 || t >= n_tokens) return;  // the GEMV wrote NaN there
  constexpr int kBatch = 16;
  float s = 0.0f;
  int sp = 0;
  for (; sp + kBatch <= splits; sp += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = partial[static_cast<int64_t>(sp + j) * plane + i];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) s += v[j];
  }
  float v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (sp + j < splits) v[j] = partial[static_cast<int64_t>(sp + j) * plane + i];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (sp + j < splits) s += v[j];
  y[i] = s;
}

}  // namespace

// Compute units of the current device (cached per device; 256 if the query fails).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// k split: the kernel keeps two workgroups resident per CU (its LDS tables),
// so workgroups run in rounds of 2 * CUs.  The number of leading workgroups
// is estimated from the pairs, assuming they spread over the experts
// (expected distinct experts of n_pairs uniform draws).  Of the split counts,
// take the one with the least rounds x (blocks per workgroup + ~2 blocks of
// fixed cost: launch, pair scan, table and pipeline fill); ties go to fewer
// splits.
GemvPlan plan_gemv(const GemvArgs& a) {
  GemvPlan pl{};
  const int nb = static_cast<int>(a.k / kQK);
  const int64_t ntiles = (a.n + kRows - 1) / kRows;
  const double ne = static_cast<double>(a.n_experts);
  const double distinct = std::min(static_cast<double>(a.n_pairs),
                                   ne * (1.0 - std::pow(1.0 - 1.0 / ne, static_cast<double>(a.n_pairs))));
  const double base_wgs = std::max(1.0, std::ceil(distinct) * static_cast<double>(ntiles));
  const double slots = 2.0 * device_cus();
  int best_splits = 1, best_bps = nb;
  double best_cost = 0.0;
  for (int splits = 1; splits <= nb; ++splits) {
    const int bps = (nb + splits - 1) / splits;
    if ((nb + bps - 1) / bps != splits) continue;  // the same split under another count
    const double rounds = std::ceil(base_wgs * splits / slots);
    const double cost = rounds * (bps + 2.0);
    if (splits == 1 || cost < best_cost) {
      best_cost = cost;
      best_splits = splits;
      best_bps = bps;
    }
  }
  pl.blocks_per_split = best_bps;
  pl.splits = best_splits;
  if (pl.splits > 1) pl.partial_bytes = static_cast<int64_t>(pl.splits) * a.n_pairs * a.n * 4;
  return pl;
}

hipError_t launch_gemv(const GemvArgs& ga, const GemvPlan& pl, void* partial, hipStream_t s) {
  if (ga.n_pairs == 0 || ga.n == 0) return hipSuccess;
  KArgs a{};
  a.w = ga.w_table;
  a.estride = ga.expert_stride;
  a.n_experts = static_cast<int>(ga.n_experts);
  a.n = static_cast<int>(ga.n);
  a.nb = static_cast<int>(ga.k / kQK);
  a.x = ga.x;
  a.xstride = ga.x_row_stride;
  a.n_tokens = static_cast<int>(ga.n_tokens);
  a.pe = ga.pair_expert;
  a.pt = ga.pair_token;
  a.n_pairs = static_cast<int>(ga.n_pairs);
  a.y = ga.y;
  a.bps = pl.blocks_per_split;
  a.splits = pl.splits;
  a.partial = static_cast<float*>(partial);
  a.ppt = ga.pairs_per_token > 0 ? static_cast<int>(ga.pairs_per_token) : 1;
  a.ff = ga.ff;
  const int ntiles = static_cast<int>((ga.n + kRows - 1) / kRows);
  const dim3 grid(ntiles, pl.splits, a.n_pairs);
  switch (ga.x_mode) {
    case kXBF16: hipLaunchKernelGGL((gemv_kernel<kXBF16>), grid, dim3(kRows), 0, s, a); break;
    case kXSwiGLU: hipLaunchKernelGGL(gemv_kernel_swiglu, grid, dim3(kRows), 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<kXF32>), grid, dim3(kRows), 0, s, a); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.splits == 1) return err;
  const int64_t plane = ga.n_pairs * ga.n;
  const int64_t grid2 = (plane + 255) / 256;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(static_cast<unsigned>(grid2)), dim3(256), 0, s, a.partial,
                     pl.splits, plane, a.pe, a.pt, a.ppt, a.n_experts, a.n_tokens, a.n, a.y);
  return hipGetLastError();
}

}  // namespace stq
