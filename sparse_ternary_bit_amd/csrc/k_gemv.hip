// Gathered STQ1_0 GEMV for the decode path: y[pair, :] = W_expert x_token.
//
// The pages say only that STQ1_0 runs through dedicated GPU kernels at about
// the speed of IQ1_M (lemmy.durstig.online post 66506, "Runtime"); the design
// below is this library's, for gfx950.
//
// Work unit: a workgroup of 256 threads owns 256 consecutive rows of one
// expert (one row per thread) and a range of 256-weight blocks along k, for
// up to kMT tokens at a time.  Every (token, expert) pair list is scanned on
// the device: the first valid pair of an expert leads, and it collects every
// later pair with that expert, so the expert's weights are streamed once per
// kMT tokens.
//
// Inner product per block: a group of four weights holds one of 32 patterns,
// so for each token and group the 32 possible signed sums of its four
// activations are tabulated in LDS once per workgroup (256 rows share each
// table).  A row then costs, per group and token, one LDS read addressed by
// the 5-bit code and one fp32 add; the block's fp16 scale multiplies the
// block sum.  Threads of a wavefront read the same group's 128-byte table at
// once, so the reads are bank-conflict free.
//
// Weights: each wavefront stages its 64 rows x 2 blocks (84 bytes per row)
// through LDS with coalesced dword loads issued one step ahead; rows are then
// read back per thread with an odd row pitch (21 dwords), which is
// conflict free.  Rows whose byte length is not a multiple of 4 use a
// per-thread direct-load variant.
//
// k split: when few experts are active, the blocks of a row are split over
// several workgroups; each writes its partial sums to scratch, and the last
// one to finish (device-scope counter) adds the partials in split order, so
// the result does not depend on scheduling.
#include <math.h>

#include <algorithm>

#include "stq_device.hpp"
#include "stq_launch.hpp"

namespace stq {
namespace {

constexpr int kRows = 256;     // rows (= threads) per workgroup
constexpr int kMT = 4;         // tokens per pass
constexpr int kStageDw = 21;   // dwords per row per staged step (2 blocks = 84 bytes)

struct KArgs {
  const uint8_t* w;
  int64_t estride;
  int n_experts;
  int n;
  int nb;          // blocks per row
  int row_dw;      // row length in dwords (staged path only)
  const void* x;
  int64_t xstride;
  int n_tokens;
  const int32_t* pe;
  const int32_t* pt;
  int n_pairs;
  float* y;
  int bps;         // blocks per split
  int splits;
  int ntiles;
  float* partial;
  unsigned* counters;
};

__device__ __forceinline__ int pair_expert(const KArgs& a, int q) { return a.pe ? a.pe[q] : 0; }
__device__ __forceinline__ int pair_token(const KArgs& a, int q) { return a.pt ? a.pt[q] : q; }

struct Shared {
  float tab[kMT][kGroups][32];                 // per token: 32 signed sums per group
  uint32_t stage[4][64 * kStageDw];            // per wavefront: 64 rows x 2 blocks
  int pairs[kMT];
  int toks[kMT];
  int mc;
  int next;
  int flag;
  unsigned long long ball[4];
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
      for (int w = 0; w < 4 && mc < kMT; ++w) {
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

// Activations of one group (4 values) of token `tok` at column `col`.
template <bool kBf16>
struct XGroup {
  uint32_t v[kBf16 ? 2 : 4];
  __device__ __forceinline__ void load(const KArgs& a, int tok, int64_t col) {
    if constexpr (kBf16) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.x) + tok * a.xstride + col);
      v[0] = p[0];
      v[1] = p[1];
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const float*>(a.x) + tok * a.xstride + col);
#pragma unroll
      for (int i = 0; i < (kBf16 ? 2 : 4); ++i) v[i] = p[i];
    }
  }
  __device__ __forceinline__ float get(int j) const {
    if constexpr (kBf16) return __uint_as_float(j & 1 ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16));
    return __uint_as_float(v[j]);
  }
};

// Table entries 8z..8z+7 of one group for zero lane z.  Entry 8z+m is the sum
// over the three kept lanes (in order) of -x or +x as bit r of m says.
__device__ __forceinline__ void build_entries(float x0, float x1, float x2, float x3, int z, float* dst) {
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
__device__ __forceinline__ void block_dot(const Shared& sh, const Block& blk, float (&acc)[kMT]) {
  const float d = half_bits_to_float(blk.d16);
  float bs[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) bs[m] = 0.0f;
  const char* tab = reinterpret_cast<const char*>(&sh.tab[0][0][0]);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t Q = blk.qs[w];
    const uint32_t Hs = blk.qh[w >> 2] << (6 - 2 * (w & 3));
    // byte j of cl / cu = 4 * code of group 8w+j / 8w+4+j
    const uint32_t cl = ((Q << 2) & 0x3C3C3C3Cu) | (Hs & 0x40404040u);
    const uint32_t cu = ((Q >> 2) & 0x3C3C3C3Cu) | ((Hs >> 1) & 0x40404040u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ol = (cl >> (8 * j)) & 0xFFu;
      const uint32_t ou = (cu >> (8 * j)) & 0xFFu;
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        const char* tm = tab + m * (kGroups * 32 * 4);
        bs[m] += *reinterpret_cast<const float*>(tm + (8 * w + j) * 128 + ol);
        bs[m] += *reinterpret_cast<const float*>(tm + (8 * w + 4 + j) * 128 + ou);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = fmaf(d, bs[m], acc[m]);
}

// Process blocks [b_begin, b_end) of this workgroup's rows for MC tokens.
// Rows past n read as zero through the buffer range check and are not stored.
template <bool kBf16, bool kStaged, int MC>
__device__ void run_chunk(const KArgs& a, Shared& sh, const uint8_t* wexp, int b_begin, int b_end,
                          float (&acc)[kMT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = tid >> 2, zi = tid & 3;  // table item of this thread: group gi, zero lane zi
  const uint32_t rb = static_cast<uint32_t>(a.nb) * kBlockBytes;

#pragma unroll
  for (int m = 0; m < kMT; ++m) acc[m] = 0.0f;

  XGroup<kBf16> xg[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) xg[m].load(a, sh.toks[m], static_cast<int64_t>(b_begin) * kQK + 4 * gi);

  if constexpr (kStaged) {
    // the wavefront's 64 rows x 84 bytes per step; dword it*64+lane of the
    // step tile is row r = idx/21, word wi = idx%21 (row pitch 21 dwords)
    const int rowbase = blockIdx.x * kRows + wave * 64;
    const int valid = max(0, min(64, a.n - rowbase));
    const uint8_t* wb = wexp + static_cast<int64_t>(rowbase) * rb + static_cast<int64_t>(b_begin) * kBlockBytes;
    const uint32_t nbytes = static_cast<uint32_t>(valid) * rb;  // rb % 4 == 0 on this path
    uint32_t voff[kStageDw];
#pragma unroll
    for (int it = 0; it < kStageDw; ++it) {
      const int idx = it * 64 + lane;
      const int r = idx / kStageDw;
      voff[it] = static_cast<uint32_t>(r) * rb + 4u * static_cast<uint32_t>(idx - r * kStageDw);
    }
    uint32_t stg[kStageDw];
    {
      const Rsrc rs = make_rsrc(wb, nbytes);
#pragma unroll
      for (int it = 0; it < kStageDw; ++it) stg[it] = buf_u32(rs, voff[it], 0);
    }
    uint32_t* st = &sh.stage[wave][0];

    for (int b0 = b_begin; b0 < b_end; b0 += 2) {
      __syncthreads();  // previous step's reads of the table and stage are done
#pragma unroll
      for (int it = 0; it < kStageDw; ++it) st[it * 64 + lane] = stg[it];
      if (b0 + 2 < b_end) {
        // move the buffer base to the next step; the range check then still
        // excludes rows past n (every offset of a valid row stays inside)
        const uint32_t shift = static_cast<uint32_t>(b0 + 2 - b_begin) * kBlockBytes;
        const Rsrc rs = make_rsrc(wb + shift, nbytes > shift ? nbytes - shift : 0u);
#pragma unroll
        for (int it = 0; it < kStageDw; ++it) stg[it] = buf_u32(rs, voff[it], 0);
      }
#pragma unroll 1
      for (int kb = 0; kb < 2; ++kb) {
        const int b = b0 + kb;
        if (kb) __syncthreads();
#pragma unroll
        for (int m = 0; m < MC; ++m)
          build_entries(xg[m].get(0), xg[m].get(1), xg[m].get(2), xg[m].get(3), zi, &sh.tab[m][gi][8 * zi]);
        if (b + 1 < b_end) {
#pragma unroll
          for (int m = 0; m < MC; ++m) xg[m].load(a, sh.toks[m], static_cast<int64_t>(b + 1) * kQK + 4 * gi);
        }
        __syncthreads();
        uint32_t v[11];
        const uint32_t* src = st + lane * kStageDw + (kb ? 10 : 0);
#pragma unroll
        for (int i = 0; i < 11; ++i) v[i] = src[i];
        const Block blk = block_from_words(v, kb != 0);
        block_dot<MC>(sh, blk, acc);
      }
    }
  } else {
    const int row = blockIdx.x * kRows + tid;
    const int64_t valid = max(0, min(kRows, a.n - static_cast<int>(blockIdx.x) * kRows));
    const uint8_t* wb = wexp + static_cast<int64_t>(blockIdx.x) * kRows * rb;
    const Rsrc rs = make_rsrc(wb, static_cast<uint32_t>((valid * rb + 3) & ~int64_t(3)));
    const uint32_t roff = static_cast<uint32_t>(row - static_cast<int>(blockIdx.x) * kRows) * rb;
    Block nxt = load_block_buf(rs, roff + static_cast<uint32_t>(b_begin) * kBlockBytes);
    for (int b = b_begin; b < b_end; ++b) {
      const Block blk = nxt;
      if (b + 1 < b_end) nxt = load_block_buf(rs, roff + static_cast<uint32_t>(b + 1) * kBlockBytes);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MC; ++m)
        build_entries(xg[m].get(0), xg[m].get(1), xg[m].get(2), xg[m].get(3), zi, &sh.tab[m][gi][8 * zi]);
      if (b + 1 < b_end) {
#pragma unroll
        for (int m = 0; m < MC; ++m) xg[m].load(a, sh.toks[m], static_cast<int64_t>(b + 1) * kQK + 4 * gi);
      }
      __syncthreads();
      block_dot<MC>(sh, blk, acc);
    }
  }
}

template <bool kBf16, bool kStaged>
__global__ __launch_bounds__(256) void gemv_kernel(KArgs a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int p = blockIdx.z;
  const int split = blockIdx.y;
  const int row = blockIdx.x * kRows + tid;
  const bool row_ok = row < a.n;

  const int e = pair_expert(a, p);
  const int tk = pair_token(a, p);
  if (e < 0 || e >= a.n_experts || tk < 0 || tk >= a.n_tokens) {
    if (split == 0 && row_ok) a.y[static_cast<int64_t>(p) * a.n + row] = __builtin_nanf("");
    return;
  }
  // lead only if no earlier valid pair uses the same expert
  if (tid == 0) sh.flag = 0;
  __syncthreads();
  for (int q = tid; q < p; q += kRows) {
    const int tq = pair_token(a, q);
    if (pair_expert(a, q) == e && tq >= 0 && tq < a.n_tokens) sh.flag = 1;
  }
  __syncthreads();
  if (sh.flag) return;

  const uint8_t* wexp = a.w + static_cast<int64_t>(e) * a.estride;
  const int b_begin = split * a.bps;
  const int b_end = min(a.nb, b_begin + a.bps);

  int cursor = p;
  for (;;) {
    gather(a, sh, e, cursor);
    const int mc = sh.mc;
    if (mc == 0) break;
    cursor = sh.next;
    float acc[kMT];
    switch (mc) {
      case 1: run_chunk<kBf16, kStaged, 1>(a, sh, wexp, b_begin, b_end, acc); break;
      case 2: run_chunk<kBf16, kStaged, 2>(a, sh, wexp, b_begin, b_end, acc); break;
      case 3: run_chunk<kBf16, kStaged, 3>(a, sh, wexp, b_begin, b_end, acc); break;
      default: run_chunk<kBf16, kStaged, 4>(a, sh, wexp, b_begin, b_end, acc); break;
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

  if (a.splits == 1) return;
  // last of the `splits` workgroups of this (expert, row tile) adds the partials in split order
  __threadfence();
  __syncthreads();
  unsigned* ctr = a.counters + static_cast<int64_t>(p) * a.ntiles + blockIdx.x;
  if (tid == 0) {
    const unsigned old = atomicAdd(ctr, 1u);
    sh.flag = (old == static_cast<unsigned>(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh.flag) return;
  __threadfence();
  cursor = p;
  for (;;) {
    gather(a, sh, e, cursor);
    const int mc = sh.mc;
    if (mc == 0) break;
    cursor = sh.next;
    if (row_ok) {
      for (int m = 0; m < mc; ++m) {
        const int64_t q = sh.pairs[m];
        float s = 0.0f;
        for (int sp = 0; sp < a.splits; ++sp)
          s += __hip_atomic_load(&a.partial[(static_cast<int64_t>(sp) * a.n_pairs + q) * a.n + row],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.y[q * a.n + row] = s;
      }
    }
    __syncthreads();
  }
  if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

GemvPlan plan_gemv(const GemvArgs& a) {
  GemvPlan pl{};
  const int nb = static_cast<int>(a.k / kQK);
  const int ntiles = static_cast<int>((a.n + kRows - 1) / kRows);
  const bool staged = (nb % 2) == 0;
  const int64_t active = std::min<int64_t>(a.n_pairs, a.n_experts);
  const int64_t base_wgs = std::max<int64_t>(1, active * ntiles);
  int64_t want = (1024 + base_wgs - 1) / base_wgs;  // aim for >= ~1024 workgroups
  const int step = staged ? 2 : 1;
  const int max_splits = (nb + step - 1) / step;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int bps = static_cast<int>((nb + want - 1) / want);
  bps = (bps + step - 1) / step * step;
  pl.blocks_per_split = bps;
  pl.splits = (nb + bps - 1) / bps;
  if (pl.splits > 1) {
    pl.partial_bytes = static_cast<int64_t>(pl.splits) * a.n_pairs * a.n * 4;
    pl.counter_bytes = a.n_pairs * ntiles * 4;
  }
  return pl;
}

hipError_t launch_gemv(const GemvArgs& ga, const GemvPlan& pl, void* counters, void* partial, hipStream_t s) {
  if (ga.n_pairs == 0 || ga.n == 0) return hipSuccess;
  KArgs a{};
  a.w = ga.w_table;
  a.estride = ga.expert_stride;
  a.n_experts = static_cast<int>(ga.n_experts);
  a.n = static_cast<int>(ga.n);
  a.nb = static_cast<int>(ga.k / kQK);
  a.row_dw = a.nb * kBlockBytes / 4;
  a.x = ga.x;
  a.xstride = ga.x_row_stride;
  a.n_tokens = static_cast<int>(ga.n_tokens);
  a.pe = ga.pair_expert;
  a.pt = ga.pair_token;
  a.n_pairs = static_cast<int>(ga.n_pairs);
  a.y = ga.y;
  a.bps = pl.blocks_per_split;
  a.splits = pl.splits;
  a.ntiles = static_cast<int>((ga.n + kRows - 1) / kRows);
  a.partial = static_cast<float*>(partial);
  a.counters = static_cast<unsigned*>(counters);
  const bool staged = (a.nb % 2) == 0;
  const dim3 grid(a.ntiles, pl.splits, a.n_pairs);
  if (ga.x_bf16) {
    if (staged) hipLaunchKernelGGL((gemv_kernel<true, true>), grid, dim3(kRows), 0, s, a);
    else hipLaunchKernelGGL((gemv_kernel<true, false>), grid, dim3(kRows), 0, s, a);
  } else {
    if (staged) hipLaunchKernelGGL((gemv_kernel<false, true>), grid, dim3(kRows), 0, s, a);
    else hipLaunchKernelGGL((gemv_kernel<false, false>), grid, dim3(kRows), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace stq
