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
// 128-byte table at once, so the reads are bank-conflict free.  With 2-4
// tokens in a pass, two tokens share an 8-byte table entry and one 8-byte
// read serves both (an LDS read issues at the same rate for 4 and 8 bytes,
// and the table reads bound the extra tokens of a pass).
// Tables are double-buffered: while block b is summed from one buffer, block
// b+1's table is built into the other, one barrier per block.
//
// Weights: the matrix is stored in 64-row tiles, block-major inside a tile,
// so a wavefront's 64 rows of block b are one contiguous 2688-byte run.  Each
// thread loads the 11 aligned words that cover its own 42-byte block with
// 16 + 16 + 12-byte buffer loads (the wavefront's loads cover the run with no
// gaps and never leave it) and realigns them with byte permutes.  Loads run
// two blocks ahead, in the order they are consumed.
//
// k split: the blocks of a row may be split over several workgroups (chosen
// per call from the expected number of active experts, see plan_gemv), and
// an expert with several tokens has each split's blocks parted further, one
// part per token up to a cap, so that every workgroup costs about the same;
// split workgroups write fp32 partial sums to scratch and a second small
// kernel adds them in k order, so the result does not depend on scheduling.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

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
// Passes of 2 or more tokens tabulate two tokens to an 8-byte entry: group g's 256-byte table at g * 256, the second pair's
// tables kPairStride further (16-byte aligned and not a multiple of 512, so
// the compiler keeps the two pairs' reads apart instead of fusing them into
// one 16-byte read that it then waits on read by read).
constexpr int kPairTab = kGroups * 32 * 8;
constexpr int kPairStride = kPairTab + 16;
static_assert(kPairStride + kPairTab <= kBufBytes, "two pair tables fit a buffer");

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
  int max_sub;     // an expert with m tokens splits each k range into min(m, max_sub) parts
  float* partial;  // [splits * max_sub, n_pairs, n] when a pair's output is split
  int32_t* pair_sub;  // per pair: its expert's part count (read by the reduction)
  int ppt;         // without pair_token: pair q uses token q / ppt
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
  int sub;
  int nsub;
  int flag;
  unsigned long long ball[kWaves];
  int wsum[kWaves];
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
      // unused token slots repeat the last token found (a 3-token pass may run as a 4-token one)
      for (int m = mc; m < kMT; ++m) sh.toks[m] = mc > 0 ? sh.toks[mc - 1] : 0;
    }
    __syncthreads();
    if (sh.mc >= kMT) break;
  }
}

// Activations of one group (4 values) of one token at column `col`, by
// source kind: fp32 rows or bf16 rows.
enum XMode { kXF32 = 0, kXBF16 = 1 };

template <int kMode>
struct XGroup {
  static constexpr int kWords = kMode == kXBF16 ? 2 : 4;
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
    }
  }
  __device__ __forceinline__ float get(int j) const {
    if constexpr (kMode == kXBF16) {
      return __uint_as_float(j & 1 ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16));
    } else {
      return __uint_as_float(v[j]);
    }
  }
};

// Signed sums of one group for zero lane z, with a, b, c its three other
// lanes in order: e[m] (m = 0..3) is a + b + c with a negated when bit 0 of
// m is set and b negated when bit 1 is.  Table entries 8z+m for m = 4..7
// (c negated as well) are the negations -e[7-m].
template <int kMode>
__device__ __forceinline__ void signed_sums(const XGroup<kMode>& xg, int z, float (&e)[4]) {
  const float x0 = xg.get(0), x1 = xg.get(1), x2 = xg.get(2), x3 = xg.get(3);
  const float a = (z == 0) ? x1 : x0;
  const float b = (z <= 1) ? x2 : x1;
  const float c = (z <= 2) ? x3 : x2;
  const float u0 = a + b;   // +a +b
  const float u1 = b - a;   // -a +b
  e[0] = u0 + c;
  e[1] = u1 + c;
  e[2] = c - u1;
  e[3] = c - u0;
}

// Table entries 8z..8z+7 of one group for zero lane z.  Entry 8z+m is the sum
// over the three kept lanes (in order) of -x or +x as bit r of m says.
template <int kMode>
__device__ __forceinline__ void build_entries(const XGroup<kMode>& xg, int z, char* dst) {
  float e[4];
  signed_sums<kMode>(xg, z, e);
  float4* o = reinterpret_cast<float4*>(dst);
  o[0] = make_float4(e[0], e[1], e[2], e[3]);
  o[1] = make_float4(-e[3], -e[2], -e[1], -e[0]);
}

// The same entries for a token pair, interleaved: entry c holds the first
// token's sum at 8c and the second's at 8c + 4.
template <int kMode>
__device__ __forceinline__ void build_pair_entries(const XGroup<kMode>& xa, const XGroup<kMode>& xb, int z,
                                                   char* dst) {
  float ea[4], eb[4];
  signed_sums<kMode>(xa, z, ea);
  signed_sums<kMode>(xb, z, eb);
  float4* o = reinterpret_cast<float4*>(dst);
  o[0] = make_float4(ea[0], eb[0], ea[1], eb[1]);
  o[1] = make_float4(ea[2], eb[2], ea[3], eb[3]);
  o[2] = make_float4(-ea[3], -eb[3], -ea[2], -eb[2]);
  o[3] = make_float4(-ea[1], -eb[1], -ea[0], -eb[0]);
}

// Pair tables: sum over the 64 groups of one block for MC = 2 or 4 tokens,
// one 8-byte read per group and token pair (an LDS read issues at the same
// rate for 4 and 8 bytes, so a token pair costs one read slot instead of
// two); a word's reads are all issued before its adds, and each token's
// sums are added in group order, as in block_dot.
template <int MC>
__device__ __forceinline__ void block_dot_pairs(const char* tab, const Block& blk, float (&acc)[kMT]) {
  constexpr int kNP = MC / 2;
  const float d = half_bits_to_float(blk.d16);
  float bs[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) bs[m] = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t Q = blk.qs[w];
    const uint32_t H = blk.qh[w >> 2];
    const int i = w & 3;
    // byte j of cl / cu = 8 * code of group 8w+j / 8w+4+j (select bit at bit 7)
    uint32_t cl = ((Q << 3) & 0x78787878u) | ((H << (7 - 2 * i)) & 0x80808080u);
    uint32_t cu = ((Q >> 1) & 0x78787878u) | ((H << (6 - 2 * i)) & 0x80808080u);
    asm("" : "+v"(cl), "+v"(cu));  // one bit-field extract per code, as in block_dot
    float2 vl[4][kNP], vu[4][kNP];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ol = __builtin_amdgcn_ubfe(cl, 8 * j, 8);
      const uint32_t ou = __builtin_amdgcn_ubfe(cu, 8 * j, 8);
#pragma unroll
      for (int p = 0; p < kNP; ++p) {
        vl[j][p] = *reinterpret_cast<const float2*>(tab + ol + (p * kPairStride + (8 * w + j) * 256));
        vu[j][p] = *reinterpret_cast<const float2*>(tab + ou + (p * kPairStride + (8 * w + 4 + j) * 256));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int p = 0; p < kNP; ++p) {
        bs[2 * p] += vl[j][p].x;
        bs[2 * p + 1] += vl[j][p].y;
        bs[2 * p] += vu[j][p].x;
        bs[2 * p + 1] += vu[j][p].y;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = fmaf(d, bs[m], acc[m]);
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

  // Table items of this thread.  Pair tables (MC = 2 or 4):
  // item (token pair tid / 256, group g, zero lane z), one per thread.  Else
  // item i = 256*m + 4*g + z for token m, items tid and tid + 512.
  constexpr bool kPair = MC >= 2;
  static_assert(!kPair || MC == 2 || MC == 4, "pair tables take 2 or 4 tokens");
  constexpr int kItems = kPair ? 128 * MC : 256 * MC;
  const int it_g = (tid >> 2) & 63, it_z = tid & 3;
  const int m0 = tid >> 8, m1 = m0 + 2;
  const bool has0 = tid < kItems, has1 = !kPair && tid + kRows < kItems;
  int tok[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) tok[m] = __builtin_amdgcn_readfirstlane(sh.toks[m]);
  // single tables: tok0 / tok1 are the tokens of items tid / tid + 512;
  // pair tables: the two tokens of this thread's pair
  int tok0 = 0, tok1 = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    if (kPair ? m == 2 * m0 : m == m0) tok0 = tok[m];
    if (kPair ? m == 2 * m0 + 1 : m == m1) tok1 = tok[m];
  }
  const int tab_off0 = kPair ? m0 * kPairStride + it_g * 256 + it_z * 64 : m0 * kTokStride + it_g * 128 + it_z * 32;
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
    if (has0) {
      x[0].load(a, tok0, col);
      if (kPair) x[1].load(a, tok1, col);
    }
    if (has1) x[1].load(a, tok1, col);
  };
  auto build = [&](const XGroup<kMode> (&x)[2], char* t) {
    if constexpr (kPair) {
      if (has0) build_pair_entries<kMode>(x[0], x[1], it_z, t + tab_off0);
    } else {
      if (has0) build_entries<kMode>(x[0], it_z, t + tab_off0);
      if (has1) build_entries<kMode>(x[1], it_z, t + tab_off1);
    }
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
    if constexpr (kPair) block_dot_pairs<MC>(tcur, blk, acc);
    else block_dot<MC>(tcur, blk, acc);
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
// pairs (gather above).  An expert with m pairs is served by min(m, max_sub)
// units, each taking one part of the workgroup's k range for all m tokens,
// so a unit costs about what a one-token expert costs whatever m is.  Units
// are numbered by leading pair in pair order (an expert's parts in k order)
// and workgroup z serves unit z, so the workgroups with work are the first
// ones launched whatever the order of the pairs: workgroups are dealt to the
// shader engines of an XCD round robin, and a periodic pattern of idle
// workgroups (pairs sorted by expert, say, with four pairs per expert) would
// otherwise put all the work on one of them.  There are at most as many
// units as valid pairs, so a grid of n_pairs workgroups covers them.
constexpr int kLeadExperts = static_cast<int>(sizeof(Shared::tab) / (2 * sizeof(int)));

__device__ __forceinline__ bool pair_valid(const KArgs& a, int q, int& e) {
  e = pair_expert(a, q);
  const int t = pair_token(a, q);
  return e >= 0 && e < a.n_experts && t >= 0 && t < a.n_tokens;
}

// With at most kLeadExperts experts: the first valid pair and the pair count
// of every expert by LDS atomics (in the table space, unused until the tables
// are built), then a running sum of the leading pairs' unit counts in pair
// order until it passes z.  Leaves the part index and count in sh.sub and
// sh.nsub.
__device__ int find_unit(const KArgs& a, Shared& sh, int z) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* first = reinterpret_cast<int*>(&sh.tab[0][0]);
  int* count = first + a.n_experts;
  const bool parts = a.max_sub > 1;  // else every leading pair is one unit and counts are not needed
  for (int e = tid; e < a.n_experts; e += kRows) {
    first[e] = 0x7FFFFFFF;
    if (parts) count[e] = 0;
  }
  if (tid == 0) sh.lead = -1;
  __syncthreads();
  for (int q = tid; q < a.n_pairs; q += kRows) {
    int e;
    if (pair_valid(a, q, e)) {
      atomicMin(&first[e], q);
      if (parts) atomicAdd(&count[e], 1);
    }
  }
  __syncthreads();
  int base = 0;
  for (int c = 0; c < a.n_pairs && base <= z; c += kRows) {
    const int q = c + tid;
    int e = -1;
    const bool lead = q < a.n_pairs && pair_valid(a, q, e) && first[e] == q;
    const int units = lead ? (parts ? min(count[e], a.max_sub) : 1) : 0;
    // inclusive prefix sum of the unit counts over the wavefront (a ballot
    // count when every count is 0 or 1), then over the waves
    int incl;
    if (parts) {
      incl = units;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
    } else {
      incl = __popcll(__ballot(lead) & (~0ull >> (63 - lane)));
    }
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int sw = sh.wsum[w];
      before += (w < wave) ? sw : 0;
      total += sw;
    }
    const int first_unit = base + before + incl - units;
    if (units > 0 && z >= first_unit && z < first_unit + units) {
      sh.lead = q;
      sh.sub = z - first_unit;
      sh.nsub = units;
    }
    base += total;
    __syncthreads();  // sh.wsum is rewritten by the next chunk
  }
  return sh.lead;  // sh.lead, sh.sub and sh.nsub are not written again in this launch
}

// Beyond kLeadExperts experts: workgroup z serves pair z, as its expert's
// only unit, if it leads (a scan of the earlier pairs), so idle workgroups
// are interleaved with busy ones.
__device__ int leader_if_first(const KArgs& a, Shared& sh, int z) {
  const int tid = threadIdx.x;
  int e;
  if (!pair_valid(a, z, e)) return -1;
  e = __builtin_amdgcn_readfirstlane(e);
  if (tid == 0) {
    sh.flag = 0;
    sh.sub = 0;
    sh.nsub = 1;
  }
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
  // this workgroup serves unit z: part `sub` of `nsub` of the expert of leading pair p
  // (uniform; p = -1 if there are fewer units)
  const int p = __builtin_amdgcn_readfirstlane(a.n_experts <= kLeadExperts ? find_unit(a, sh, z)
                                                                             : leader_if_first(a, sh, z));
  if (p < 0) return;
  const int e = __builtin_amdgcn_readfirstlane(pair_expert(a, p));
  const bool parts = a.max_sub > 1;
  const int sub = parts ? __builtin_amdgcn_readfirstlane(sh.sub) : 0;
  const int nsub = parts ? __builtin_amdgcn_readfirstlane(sh.nsub) : 1;

  const uint8_t* wexp = a.w + static_cast<int64_t>(e) * a.estride;
  // blocks of split `split`, then part `sub` of them (a part is empty only when the last
  // split is shorter than nsub: its workgroup then adds zeros to its slot)
  const int s_begin = split * a.bps;
  const int s_len = min(a.nb, s_begin + a.bps) - s_begin;
  const int b_begin = parts ? s_begin + (sub * s_len) / nsub : s_begin;
  const int b_end = parts ? s_begin + ((sub + 1) * s_len) / nsub : s_begin + s_len;
  // partial slot of this unit: k order is split-major, part-minor
  const int n_slots = a.splits * nsub;
  const int slot = split * nsub + sub;

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
      case 3:  // pair tables take 3 tokens as 4 (the fourth repeats the third, its sums unused)
        run_chunk<kMode, 4>(a, sh, wexp, b_begin, b_end, acc);
        break;
      default: run_chunk<kMode, 4>(a, sh, wexp, b_begin, b_end, acc); break;
    }
    if (row_ok) {
#pragma unroll
      for (int m = 0; m < kMT; ++m) {
        if (m < mc) {
          const int64_t q = sh.pairs[m];
          if (n_slots == 1) a.y[q * a.n + row] = acc[m];
          else a.partial[(static_cast<int64_t>(slot) * a.n_pairs + q) * a.n + row] = acc[m];
        }
      }
    }
    // the reduction learns each pair's part count from the first unit of its expert
    if (a.pair_sub && split == 0 && sub == 0 && blockIdx.x == 0 && tid < mc) a.pair_sub[sh.pairs[tid]] = nsub;
    __syncthreads();  // sh.pairs is rewritten by the next gather
  }
}

// At most 128 VGPRs (4 waves per SIMD, two workgroups per CU as the LDS
// allows); the fp32-row kernel's pair-table builds need a few bytes of
// spill outside the block loop to stay there.
template <int kMode>
__global__ __launch_bounds__(kRows, 4) void gemv_kernel(KArgs a) {
  gemv_main<kMode>(a);
}

// y[p, r] = sum over the pair's slots s, in order, of partial[s, p, r], for
// valid pairs whose output is split (splits x the pair's part count > 1; the
// others were written directly).  Workgroup (x, p) covers rows 256x.. of
// pair p, so the pair's checks and slot count are uniform.  The first 16 of
// the max_slots allocated slots are loaded before the pair's ids and part
// count arrive (every allocated slot is in bounds; the ones past the pair's
// count are not used), so a call with at most 16 slots pays one memory
// latency for its data; the additions stay in slot (= k) order.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ partial, int splits,
                                                            int max_slots, const int32_t* __restrict__ pair_sub,
                                                            int n_pairs, const int32_t* __restrict__ pe,
                                                            const int32_t* __restrict__ pt, int ppt, int n_experts,
                                                            int n_tokens, int n, float* __restrict__ y) {
  const int p = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n) return;
  const int64_t plane = static_cast<int64_t>(n_pairs) * n;
  const int64_t i = static_cast<int64_t>(p) * n + r;
  constexpr int kBatch = 16;
  float v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (j < max_slots) v[j] = partial[static_cast<int64_t>(j) * plane + i];
  const int e = pe ? pe[p] : 0;
  const int t = pt ? pt[p] : p / ppt;
  if (e < 0 || e >= n_experts || t < 0 || t >= n_tokens) return;  // the GEMV wrote NaN there
  const int slots = pair_sub ? splits * pair_sub[p] : splits;
  if (slots == 1) return;  // the GEMV wrote y itself
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (j < slots) s += v[j];
  for (int sp = kBatch; sp < slots; sp += kBatch) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (sp + j < slots) v[j] = partial[static_cast<int64_t>(sp + j) * plane + i];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (sp + j < slots) s += v[j];
  }
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

// Work of one pass over a block, relative to a one-token pass, for a pass
// of 1..4 tokens (measured with bf16 activations on a full layer, every
// expert given the same token count: 1, 1.45, 2.1 and 2.18); an expert with
// m tokens makes floor(m / 4) four-token passes and one pass of the rest.
static double block_cost(int m) {
  constexpr double kPass[5] = {0.0, 1.0, 1.45, 2.1, 2.18};
  return (m / 4) * kPass[4] + kPass[m % 4];
}

// k split: the kernel keeps two workgroups resident per CU (its LDS tables),
// so workgroups run in rounds of 2 * CUs.  Each split's blocks are parted
// further by token count (an expert with m pairs takes min(m, sub) units,
// sub <= max_sub keeping at least kMinSubBlocks blocks a part), so heavy
// experts need not hold the last round.  For each (splits, max_sub) the
// time is estimated in one-token block passes from the expected experts per
// token count (pairs spread uniformly over the experts, m binomial): the
// units' work plus kUnitCost per unit (launch, pair scan, table and pipeline
// fill) spread over the resident slots, but no less than the longest unit,
// plus a fraction of the longest unit for the tail, plus the fp32 partial
// sums' write and read at the rate the slots stream weights.  The constants
// fit measured times of a 256-expert 4096 x 7168 layer at 4 to 512 pairs.
// Plans whose partial sums pass kMaxPartialBytes are not taken (one k split
// and one part per expert needs none).
constexpr int kMinSubBlocks = 4;
constexpr int kMaxSub = 8;
constexpr double kUnitCost = 3.5;
constexpr double kTailShare = 0.2;
constexpr double kMaxPartialBytes = 1024.0 * 1024.0 * 1024.0;

static void estimate_plan(const GemvArgs& a, int cus, int& best_splits, int& best_bps, int& best_sub) {
  const int nb = static_cast<int>(a.k / kQK);
  const double ntiles = static_cast<double>((a.n + kRows - 1) / kRows);
  const bool parts_ok = a.n_experts <= kLeadExperts;  // beyond, an expert is one unit
  const double slots = 2.0 * cus;
  // expected number of experts with exactly m pairs, over m within 8 standard
  // deviations of the mean (binomial in log space, so nothing underflows)
  std::vector<std::pair<int, double>> cnt;
  const double np = static_cast<double>(a.n_pairs), ne = static_cast<double>(a.n_experts);
  if (a.n_experts <= 1) {
    cnt.emplace_back(static_cast<int>(a.n_pairs), 1.0);
  } else {
    const double p = 1.0 / ne, mean = np * p, sd = std::sqrt(np * p * (1.0 - p));
    const int lo = std::max(1, static_cast<int>(std::floor(mean - 8.0 * sd)) - 1);
    const int hi = static_cast<int>(std::min(np, std::ceil(mean + 8.0 * sd) + 8.0));
    const double lg_n = std::lgamma(np + 1.0), lp = std::log(p), lq = std::log1p(-p);
    for (int m = lo; m <= hi; ++m) {
      const double lpm = lg_n - std::lgamma(m + 1.0) - std::lgamma(np - m + 1.0) + m * lp + (np - m) * lq;
      const double c = ne * std::exp(lpm);
      if (c > 1e-9) cnt.emplace_back(m, c);
    }
  }
  best_splits = 1;
  best_bps = nb;
  best_sub = 1;
  double best_cost = -1.0;
  for (int splits = 1; splits <= nb; ++splits) {
    const int bps = (nb + splits - 1) / splits;
    if ((nb + bps - 1) / bps != splits) continue;  // the same split under another count
    const int sub_cap = parts_ok ? std::max(1, std::min(kMaxSub, bps / kMinSubBlocks)) : 1;
    for (int max_sub = 1; max_sub <= sub_cap; ++max_sub) {
      const double n_slots = static_cast<double>(splits) * max_sub;
      if (n_slots > 1.0 && n_slots * np * static_cast<double>(a.n) * 4.0 > kMaxPartialBytes) continue;
      double work = 0.0, longest = 0.0, partial_sums = 0.0;
      for (const auto& [m, count] : cnt) {
        const int parts = std::min(m, max_sub);
        const double c = block_cost(m) * bps;
        work += count * (c + kUnitCost * parts);
        if (count >= 0.3) longest = std::max(longest, c / parts + kUnitCost);
        if (splits * parts > 1) partial_sums += m * count * splits * parts;  // pair outputs through scratch
      }
      work *= ntiles * splits;
      const double traffic = partial_sums * static_cast<double>(a.n) * 8.0 / (slots * kRows * kBlockBytes);
      const double cost = std::max(work / slots, longest) + kTailShare * longest + traffic;
      if (best_cost < 0.0 || cost < best_cost * (1.0 - 1e-9)) {
        best_cost = cost;
        best_splits = splits;
        best_bps = bps;
        best_sub = max_sub;
      }
    }
  }
}

// The estimate depends only on the shapes and the CU count; decode loops
// repeat a few shapes, so each host thread keeps its last 16 answers.
GemvPlan plan_gemv(const GemvArgs& a, int for_cus) {
  struct Entry {
    int64_t n_pairs, n_experts, n, k;
    int cus, splits, bps, sub;
  };
  thread_local Entry cache[16];
  thread_local int cache_used = 0, cache_next = 0;
  const int cus = for_cus > 0 ? for_cus : device_cus();
  const int nb = static_cast<int>(a.k / kQK);
  const bool parts_ok = a.n_experts <= kLeadExperts;
  int best_splits = 0, best_bps = 0, best_sub = 0;
  for (int i = 0; i < cache_used; ++i) {
    const Entry& c = cache[i];
    if (c.n_pairs == a.n_pairs && c.n_experts == a.n_experts && c.n == a.n && c.k == a.k && c.cus == cus) {
      best_splits = c.splits;
      best_bps = c.bps;
      best_sub = c.sub;
      break;
    }
  }
  if (best_splits == 0) {
    estimate_plan(a, cus, best_splits, best_bps, best_sub);
    cache[cache_next] = Entry{a.n_pairs, a.n_experts, a.n, a.k, cus, best_splits, best_bps, best_sub};
    cache_next = (cache_next + 1) % 16;
    cache_used = std::min(cache_used + 1, 16);
  }
  GemvPlan pl{};
  // STQ_GEMV_PLAN="splits,max_sub" replaces the estimate (tuning and tests;
  // max_sub may exceed the blocks of a split, leaving some parts empty)
  if (const char* ev = std::getenv("STQ_GEMV_PLAN")) {
    int sp = 0, ms = 0;
    if (std::sscanf(ev, "%d,%d", &sp, &ms) == 2 && sp >= 1 && sp <= nb && ms >= 1 && ms <= kMaxSub) {
      best_bps = (nb + sp - 1) / sp;
      best_splits = (nb + best_bps - 1) / best_bps;
      best_sub = parts_ok ? ms : 1;
    }
  }
  pl.blocks_per_split = best_bps;
  pl.splits = best_splits;
  pl.max_sub = best_sub;
  const int64_t n_slots = static_cast<int64_t>(pl.splits) * pl.max_sub;
  if (n_slots > 1) {
    pl.partial_floats = n_slots * a.n_pairs * a.n;
    pl.partial_bytes = (pl.partial_floats * 4 + 255) / 256 * 256 + (pl.max_sub > 1 ? a.n_pairs * 4 : 0);
  }
  return pl;
}

static int32_t* pair_sub_of(const GemvPlan& pl, void* partial) {
  return pl.max_sub > 1
             ? reinterpret_cast<int32_t*>(static_cast<char*>(partial) + (pl.partial_floats * 4 + 255) / 256 * 256)
             : nullptr;
}

GemvPartials gemv_partials(const GemvPlan& pl, void* partial) {
  GemvPartials g{};
  if (pl.partial_bytes > 0) {
    g.partial = static_cast<const float*>(partial);
    g.splits = pl.splits;
    g.max_slots = pl.splits * pl.max_sub;
    g.pair_sub = pair_sub_of(pl, partial);
  }
  return g;
}

hipError_t launch_gemv(const GemvArgs& ga, const GemvPlan& pl, void* partial, hipStream_t s, bool reduce) {
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
  a.max_sub = pl.max_sub;
  a.partial = static_cast<float*>(partial);
  a.pair_sub = pair_sub_of(pl, partial);
  a.ppt = ga.pairs_per_token > 0 ? static_cast<int>(ga.pairs_per_token) : 1;
  const int ntiles = static_cast<int>((ga.n + kRows - 1) / kRows);
  const dim3 grid(ntiles, pl.splits, a.n_pairs);
  switch (ga.x_mode) {
    case kXBF16: hipLaunchKernelGGL((gemv_kernel<kXBF16>), grid, dim3(kRows), 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<kXF32>), grid, dim3(kRows), 0, s, a); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.partial_bytes == 0 || !reduce) return err;
  const dim3 grid2(static_cast<unsigned>((ga.n + 255) / 256), static_cast<unsigned>(ga.n_pairs));
  hipLaunchKernelGGL(reduce_splits_kernel, grid2, dim3(256), 0, s, a.partial, pl.splits, pl.splits * pl.max_sub,
                     a.pair_sub, a.n_pairs, a.pe, a.pt, a.ppt, a.n_experts, a.n_tokens, a.n, a.y);
  return hipGetLastError();
}

}  // namespace stq
