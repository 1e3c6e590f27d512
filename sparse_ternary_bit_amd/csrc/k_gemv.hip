// Gathered STQ1_0 GEMV for the decode path: y[pair, :] = W_expert x_token.
//
// The pages say only that STQ1_0 runs through dedicated GPU kernels at about
// the speed of IQ1_M (lemmy.durstig.online post 66506, "Runtime"); the design
// below is this library's, for gfx950.
//
// Work unit: a workgroup of 512 threads owns 512 consecutive rows of one
// expert (one row per thread, eight 64-row tiles) and a range of 256-weight
// blocks along k, for up to kMT tokens at a time (kMT2 on the matrix
// cores).  The (token, expert) pair list is scanned on the device: the first
// valid pair of an expert leads and collects every later pair with that
// expert, so the expert's weights stream once per pass.
//
// Inner product per block: a group of four weights holds one of 32 patterns,
// so for each token and group the 32 possible signed sums of its four
// activations are tabulated in LDS once per workgroup (512 rows share each
// table).  A row then costs, per group, one bit-field extract of its 5-bit
// code (already scaled by 4) and, per token, one LDS read with the group's
// table offset as an immediate plus one fp32 add; the block's fp16 scale
// multiplies the block sum.  All threads of a wavefront read the same group's
// 128-byte table at once, so the reads are bank-conflict free.  Group tables
// sit 16 bytes more than their size apart, so that the 16-byte stores that
// build them (a wavefront writes 16 neighbouring groups' tables at once) fall
// on all eight 16-byte bank groups instead of two or four.  With 2-4
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
// one block ahead, in the order they are consumed.
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
constexpr int kMT = 4;                     // tokens per table pass
constexpr int kMT2 = 2 * kMT;              // tokens per matrix-core pass
// One-token passes: group g's 128-byte table at g * kGrp1.
constexpr int kGrp1 = 32 * 4 + 16;
constexpr int kTabBytes = kGroups * kGrp1;
// Passes of 2 or more tokens tabulate two tokens to an 8-byte entry: group
// g's 256-byte table at g * kGrp2, the second pair's tables kPairStride
// further (16-byte aligned and not a multiple of 512, so the compiler keeps
// the two pairs' reads apart instead of fusing them into one 16-byte read
// that it then waits on read by read).
constexpr int kGrp2 = 32 * 8 + 16;
constexpr int kPairTab = kGroups * kGrp2;
constexpr int kPairStride = kPairTab + 16;
constexpr int kBufBytes = kPairStride + kPairTab;  // one table buffer
static_assert(kTabBytes <= kBufBytes && kPairStride % 512 != 0, "table layout");

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
  int order;       // number units by cost class (longest first) when the pairs fit one chunk
};

// bf16 passes of at least this many tokens run on the matrix cores (in the
// kernel variant that has that form; fewer tokens use the tables)
constexpr int kMfmaMinTokens = 3;

__device__ __forceinline__ int pair_expert(const KArgs& a, int q) { return a.pe ? a.pe[q] : 0; }
__device__ __forceinline__ int pair_token(const KArgs& a, int q) { return a.pt ? a.pt[q] : q / a.ppt; }

struct Shared {
  // bf16 pattern table of the matrix-core form: entry c of lut[0..31] holds
  // lanes 0,1 of code c, entry c of lut[32..63] lanes 2,3 (two 4-byte reads
  // 128 bytes apart are bank-conflict free whatever the codes)
  uint32_t lut[64];
  alignas(16) char tab[2][kBufBytes];       // two table buffers; per token 32 signed sums x 64 groups
  int pairs[kMT2];
  int toks[kMT2];
  int mc;
  int next;
  int lead;
  int sub;
  int nsub;
  int lead_m;  // valid pairs of the lead's expert when the search counted them, else 0
  int flag;
  unsigned long long ball[kWaves];
  int wsum[kWaves];
};

// Collect up to kCap pairs with expert e and a valid token, from `cursor` on,
// in index order.  Leaves the count in sh.mc and the resume index in sh.next.
// Each matching thread places its own pair and token at its rank among the
// matches (a prefix count over the wavefronts' ballots), so no thread loads
// the pairs one after another.
template <int kCap>
__device__ void gather(const KArgs& a, Shared& sh, int e, int cursor) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mc = 0;  // pairs found so far, the same in every thread
  for (int base = cursor; base < a.n_pairs && mc < kCap; base += kRows) {
    const int q = base + tid;
    bool match = false;
    int tq = 0;
    if (q < a.n_pairs) {
      tq = pair_token(a, q);
      match = pair_expert(a, q) == e && tq >= 0 && tq < a.n_tokens;
    }
    const unsigned long long bal = __ballot(match);
    if (lane == 0) sh.ball[wave] = bal;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = __popcll(sh.ball[w]);
      before += (w < wave) ? c : 0;
      total += c;
    }
    const int slot = mc + before + __popcll(bal & ((1ull << lane) - 1ull));
    if (match && slot < kCap) {
      sh.pairs[slot] = q;
      sh.toks[slot] = tq;
      // the pass is full: the next one resumes after its last pair
      if (slot == kCap - 1) sh.next = q + 1;
    }
    mc = min(kCap, mc + total);
    __syncthreads();  // sh.ball is rewritten by the next chunk; the slots are visible
  }
  if (tid == 0) {
    sh.mc = mc;
    if (mc < kCap) sh.next = a.n_pairs;  // every remaining pair was scanned
    // unused token slots repeat the last token found (a 3-token pass may run as a 4-token one)
    for (int m = mc; m < kCap; ++m) sh.toks[m] = mc > 0 ? sh.toks[mc - 1] : 0;
  }
  __syncthreads();
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
        vl[j][p] = *reinterpret_cast<const float2*>(tab + ol + (p * kPairStride + (8 * w + j) * kGrp2));
        vu[j][p] = *reinterpret_cast<const float2*>(tab + ou + (p * kPairStride + (8 * w + 4 + j) * kGrp2));
      }
    }
    // keep the word's reads ahead of its adds and the next word's reads
    // behind them (hoisting several words' reads runs out of registers and
    // forces waits for every read in flight)
    __builtin_amdgcn_sched_barrier(0);
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
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = fmaf(d, bs[m], acc[m]);
}

// Sum over the 64 groups of one block of table[code], for MC tokens.  A code
// word's 8 table reads per token are all issued before its adds (left to
// itself the scheduler may interleave each read with its add and wait on
// every read).  Each token's sums are added in group order.
template <int MC>
__device__ __forceinline__ void block_dot(const char* tab, const Block& blk, float (&acc)[kMT]) {
  static_assert(MC * kTabBytes <= kBufBytes, "one-token tables of the pass fit a buffer");
  const float d = half_bits_to_float(blk.d16);
  float bs[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) bs[m] = 0.0f;
  // word w's reads: v[m][2j] for group 8w+j, v[m][2j+1] for group 8w+4+j
  auto reads = [&](int w, float (&v)[MC][8]) {
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
        v[m][2 * j] = *reinterpret_cast<const float*>(tab + ol + (m * kTabBytes + (8 * w + j) * kGrp1));
        v[m][2 * j + 1] = *reinterpret_cast<const float*>(tab + ou + (m * kTabBytes + (8 * w + 4 + j) * kGrp1));
      }
    }
  };
  auto adds = [&](const float (&v)[MC][8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        bs[m] += v[m][2 * j];
        bs[m] += v[m][2 * j + 1];
      }
  };
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float v[MC][8];
    reads(w, v);
    __builtin_amdgcn_sched_barrier(0);
    adds(v);
    __builtin_amdgcn_sched_barrier(0);
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

  // Table items of this thread.  Pair tables (MC = 2 or 4): item (token pair
  // tid / 256, group g, zero lane z).  One token (MC = 1): item (g, z) of the
  // token, threads 0..255.
  constexpr bool kPair = MC >= 2;
  static_assert(MC == 1 || MC == 2 || MC == 4, "one-token tables or pair tables of 2 or 4 tokens");
  constexpr int kItems = kPair ? 128 * MC : 256;
  const int it_g = (tid >> 2) & 63, it_z = tid & 3;
  const int m0 = tid >> 8;
  const bool has0 = tid < kItems;
  int tok[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) tok[m] = __builtin_amdgcn_readfirstlane(sh.toks[m]);
  // the token (one-token tables) or the two tokens of this thread's pair
  int tok0 = 0, tok1 = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    if (kPair ? m == 2 * m0 : m == 0) tok0 = tok[m];
    if (kPair && m == 2 * m0 + 1) tok1 = tok[m];
  }
  const int tab_off0 = kPair ? m0 * kPairStride + it_g * kGrp2 + it_z * 64 : it_g * kGrp1 + it_z * 32;

#pragma unroll
  for (int m = 0; m < kMT; ++m) acc[m] = 0.0f;
  // an empty part (uniform over the workgroup) adds zeros; the loads below
  // assume b_begin < b_end
  if (b_begin >= b_end) return;

  // this wavefront's rows are one tile of the packed matrix
  const int rowbase = blockIdx.x * kRows + wave * 64;
  const int valid = max(0, min(kTileRows, a.n - rowbase));
  const uint8_t* tb = wexp + static_cast<int64_t>(min(rowbase, a.n)) * a.nb * kBlockBytes;
  const uint32_t tile_bytes = (static_cast<uint32_t>(valid) * a.nb * kBlockBytes + 3u) & ~3u;
  const Rsrc rs = make_rsrc(tb, tile_bytes);
  // a block past b_end is "loaded" from the end of the tile's range, where the
  // range check returns zeros without a memory access: the load stays
  // unconditional (a skipped load makes the compiler copy the previous block
  // into the load's registers first)
  auto load_w = [&](RawBlock& r, int b) {
    const uint32_t off = b < b_end ? (static_cast<uint32_t>(b) * valid + lane) * kBlockBytes : tile_bytes;
    load_raw_block(rs, off, r);
  };
  // every thread loads (threads without a table item load token 0's group)
  auto load_x = [&](XGroup<kMode> (&x)[2], int b) {
    const int64_t col = static_cast<int64_t>(b) * kQK + 4 * it_g;
    x[0].load(a, tok0, col);
    if (kPair) x[1].load(a, tok1, col);
  };
  auto build = [&](const XGroup<kMode> (&x)[2], char* t) {
    if constexpr (kPair) {
      if (has0) build_pair_entries<kMode>(x[0], x[1], it_z, t + tab_off0);
    } else {
      if (has0) build_entries<kMode>(x[0], it_z, t + tab_off0);
    }
  };
  // 42*(b*valid + lane) is 2 mod 4 exactly when b*valid + lane is odd
  const bool lane_odd = (lane & 1) != 0;
  char* buf0 = sh.tab[0];
  char* buf1 = sh.tab[1];

  // Pipeline over blocks: while block b is multiplied, the weights of block
  // b+1 and the activations of block b+2 are in flight, and table b+1 is
  // built from activations loaded one block earlier.  Each stream has one
  // register set: a load reuses the registers its predecessor was read from,
  // so no copy of an in-flight load (which would wait for it) is needed.
  RawBlock w;
  XGroup<kMode> xn[2];
  auto step = [&](char* tcur, char* tnext, int b) {
    const bool odd = ((static_cast<uint32_t>(b) * valid) & 1u) ? !lane_odd : lane_odd;
    const Block blk = realign_block(w, odd);
    __builtin_amdgcn_sched_barrier(0);
    load_w(w, b + 1);
    if (b + 1 < b_end) build(xn, tnext);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xn, min(b + 2, b_end - 1));
    if constexpr (kPair) block_dot_pairs<MC>(tcur, blk, acc);
    else block_dot<MC>(tcur, blk, acc);
    __syncthreads();  // table b+1 is complete and every thread is done with table b
  };
  {
    load_w(w, b_begin);
    XGroup<kMode> x0[2];
    load_x(x0, b_begin);
    load_x(xn, min(b_begin + 1, b_end - 1));
    build(x0, buf0);
    __syncthreads();
  }
  for (int b = b_begin; b < b_end; b += 2) {
    step(buf0, buf1, b);
    if (b + 1 < b_end) step(buf1, buf0, b + 1);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One block of this thread's row for a set of four tokens on the matrix
// cores.  v_mfma_f32_4x4x4_16b_bf16 multiplies 16 independent 4x4 blocks;
// here block b is the wavefront's row quad 4b..4b+3 and k is one group: the B
// operand of lane l is row l's four weights of the group (a pattern read
// from the bf16 table), the A operand is the group's four activations of
// tokens 0..3, which the instruction broadcasts from one block to all 16
// (cbsz 4, abid): lane 4b+i holds token i's activations of group 16s+b for
// s = 0..3, so four 8-byte reads per block fetch all 64 groups.  Lane l's
// four results are row l for tokens 0..3.  Products of bf16 values are exact
// in fp32; the group sums accumulate in fp32 (even and odd groups apart),
// then the block's d scales them (one FMA per token), as in block_dot.  A
// pass of 5-8 tokens runs two sets on the same pattern reads, so the
// weights stream once for eight tokens.
// Group G's product: the activations of group G (block G % 16 of the set
// G / 16) broadcast to all 16 blocks.  abid must be an immediate, hence the
// template.
template <int G>
__device__ __forceinline__ f32x4_t mfma_group(const s16x4_t (&xa)[4], s16x4_t w, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xa[G >> 4], w, c, 4, G & 15, 0);
}

// Code word W (groups 8W..8W+7) of one block: the pattern reads, bl for the
// four low-nibble groups and bu for the four high-nibble ones.
template <int W>
__device__ __forceinline__ void word_patterns(const Block& blk, const char* lb, s16x4_t (&bl)[4], s16x4_t (&bu)[4]) {
  const uint32_t Q = blk.qs[W];
  const uint32_t Hs = blk.qh[W >> 2] << (6 - 2 * (W & 3));
  // byte j of cl / cu = 4 * code of group 8W+j / 8W+4+j
  uint32_t cl = ((Q << 2) & 0x3C3C3C3Cu) | (Hs & 0x40404040u);
  uint32_t cu = ((Q >> 2) & 0x3C3C3C3Cu) | ((Hs >> 1) & 0x40404040u);
  asm("" : "+v"(cl), "+v"(cu));  // one bit-field extract per code, as in block_dot
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t ol = __builtin_amdgcn_ubfe(cl, 8 * j, 8);
    const uint32_t ou = __builtin_amdgcn_ubfe(cu, 8 * j, 8);
    const uint64_t l0 = *reinterpret_cast<const uint32_t*>(lb + ol);
    const uint64_t l1 = *reinterpret_cast<const uint32_t*>(lb + ol + 128);
    const uint64_t u0 = *reinterpret_cast<const uint32_t*>(lb + ou);
    const uint64_t u1 = *reinterpret_cast<const uint32_t*>(lb + ou + 128);
    bl[j] = __builtin_bit_cast(s16x4_t, (l1 << 32) | l0);
    bu[j] = __builtin_bit_cast(s16x4_t, (u1 << 32) | u0);
  }
}

// The MFMAs of code word W for each token set: its low-nibble groups into
// c[t][0], high into c[t][1] (the same instruction order for every set, so a
// token's result does not depend on the set it is in).
template <int W, int kSets>
__device__ __forceinline__ void word_mfmas(const s16x4_t (&xa)[kSets][4], const s16x4_t (&bl)[4],
                                           const s16x4_t (&bu)[4], f32x4_t (&c)[kSets][2]) {
#pragma unroll
  for (int t = 0; t < kSets; ++t) {
    c[t][0] = mfma_group<8 * W + 0>(xa[t], bl[0], c[t][0]);
    c[t][1] = mfma_group<8 * W + 4>(xa[t], bu[0], c[t][1]);
    c[t][0] = mfma_group<8 * W + 1>(xa[t], bl[1], c[t][0]);
    c[t][1] = mfma_group<8 * W + 5>(xa[t], bu[1], c[t][1]);
    c[t][0] = mfma_group<8 * W + 2>(xa[t], bl[2], c[t][0]);
    c[t][1] = mfma_group<8 * W + 6>(xa[t], bu[2], c[t][1]);
    c[t][0] = mfma_group<8 * W + 3>(xa[t], bl[3], c[t][0]);
    c[t][1] = mfma_group<8 * W + 7>(xa[t], bu[3], c[t][1]);
  }
}

// Words W and up: the pattern reads of word W+1 are issued before the MFMAs
// of word W, so the reads of one word are in flight while the previous
// word's products run.
template <int W, int kSets>
__device__ __forceinline__ void words_from(const Block& blk, const char* lb, const s16x4_t (&xa)[kSets][4],
                                           s16x4_t (&bl)[4], s16x4_t (&bu)[4], f32x4_t (&c)[kSets][2]) {
  if constexpr (W < 7) {
    s16x4_t nl[4], nu[4];
    word_patterns<W + 1>(blk, lb, nl, nu);
    word_mfmas<W, kSets>(xa, bl, bu, c);
    words_from<W + 1, kSets>(blk, lb, xa, nl, nu, c);
  } else {
    word_mfmas<W, kSets>(xa, bl, bu, c);
  }
}

// One block for kSets sets of four tokens; set t's activations are staged
// 2048 bytes after set t-1's.  The pattern reads serve every set.
template <int kSets>
__device__ __forceinline__ void block_mfma(const char* xs, const uint32_t* lut, const Block& blk, int lane,
                                           float (&acc)[kMT * kSets]) {
  const float d = half_bits_to_float(blk.d16);
  s16x4_t xa[kSets][4];
#pragma unroll
  for (int t = 0; t < kSets; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[t][s] = *reinterpret_cast<const s16x4_t*>(xs + t * 2048 + (64 * s + lane) * 8);
  f32x4_t c[kSets][2];
#pragma unroll
  for (int t = 0; t < kSets; ++t) c[t][0] = c[t][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const char* lb = reinterpret_cast<const char*>(lut);
  s16x4_t bl[4], bu[4];
  word_patterns<0>(blk, lb, bl, bu);
  words_from<0, kSets>(blk, lb, xa, bl, bu, c);
#pragma unroll
  for (int t = 0; t < kSets; ++t)
#pragma unroll
    for (int m = 0; m < kMT; ++m) acc[kMT * t + m] = fmaf(d, c[t][0][m] + c[t][1][m], acc[kMT * t + m]);
}

// Blocks [b_begin, b_end) of this workgroup's rows for bf16 activations and
// up to 4 * kSets tokens on the matrix cores (token slots past the pass's
// count repeat its last token; their results are not stored).  The pipeline
// is run_chunk's: weights one block ahead, activations two; each block's
// activations (4 tokens x 64 groups x 8 bytes per set) are staged in LDS in
// [set][group][token] order while the previous block is multiplied.
template <int kSets>
__device__ __forceinline__ void run_chunk_mfma(const KArgs& a, Shared& sh, const uint8_t* wexp, int b_begin,
                                               int b_end, float (&acc)[kMT * kSets]) {
  constexpr int kTok = kMT * kSets;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // staging item of this thread (threads 0..64 * kTok - 1): token tid >> 6, group tid & 63
  const int st_m = tid >> 6, st_g = tid & 63;
  const bool stages = tid < kTok * 64;
  int tok_st = 0;
#pragma unroll
  for (int m = 0; m < kTok; ++m) {
    const int t = __builtin_amdgcn_readfirstlane(sh.toks[m]);
    if (m == st_m) tok_st = t;
  }
  const int st_off = (st_m >> 2) * 2048 + (st_g * 4 + (st_m & 3)) * 8;

#pragma unroll
  for (int m = 0; m < kTok; ++m) acc[m] = 0.0f;
  if (b_begin >= b_end) return;  // an empty part, as in run_chunk

  const int rowbase = blockIdx.x * kRows + wave * 64;
  const int valid = max(0, min(kTileRows, a.n - rowbase));
  const uint8_t* tb = wexp + static_cast<int64_t>(min(rowbase, a.n)) * a.nb * kBlockBytes;
  const uint32_t tile_bytes = (static_cast<uint32_t>(valid) * a.nb * kBlockBytes + 3u) & ~3u;
  const Rsrc rs = make_rsrc(tb, tile_bytes);
  // a block past b_end is "loaded" from the end of the tile's range, where the
  // range check returns zeros without a memory access: the load stays
  // unconditional (a skipped load makes the compiler copy the previous block
  // into the load's registers first)
  auto load_w = [&](RawBlock& r, int b) {
    const uint32_t off = b < b_end ? (static_cast<uint32_t>(b) * valid + lane) * kBlockBytes : tile_bytes;
    load_raw_block(rs, off, r);
  };
  // every thread loads (threads that stage nothing load token 0's group)
  auto load_x = [&](XGroup<kXBF16>& x, int b) { x.load(a, tok_st, static_cast<int64_t>(b) * kQK + 4 * st_g); };
  auto stage = [&](const XGroup<kXBF16>& x, char* t) {
    if (stages) *reinterpret_cast<uint2*>(t + st_off) = make_uint2(x.v[0], x.v[1]);
  };
  const bool lane_odd = (lane & 1) != 0;
  char* buf0 = sh.tab[0];
  char* buf1 = sh.tab[1];

  // one register set per stream, as in run_chunk
  RawBlock w;
  XGroup<kXBF16> xn;
  auto step = [&](char* tcur, char* tnext, int b) {
    const bool odd = ((static_cast<uint32_t>(b) * valid) & 1u) ? !lane_odd : lane_odd;
    const Block blk = realign_block(w, odd);
    __builtin_amdgcn_sched_barrier(0);
    load_w(w, b + 1);
    if (b + 1 < b_end) stage(xn, tnext);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xn, min(b + 2, b_end - 1));
    block_mfma<kSets>(tcur, sh.lut, blk, lane, acc);
    __syncthreads();  // block b+1's activations are staged and every thread is done with block b's
  };
  {
    load_w(w, b_begin);
    XGroup<kXBF16> x0;
    load_x(x0, b_begin);
    load_x(xn, min(b_begin + 1, b_end - 1));
    stage(x0, buf0);
    __syncthreads();
  }
  for (int b = b_begin; b < b_end; b += 2) {
    step(buf0, buf1, b);
    if (b + 1 < b_end) step(buf1, buf0, b + 1);
  }
}

// A pair leads when its token is valid and no earlier valid pair names the
// same expert; the leading pair of an expert collects all of that expert's
// pairs (gather above).  An expert with m pairs is served by min(m, max_sub)
// units, each taking one part of the workgroup's k range for all m tokens,
// so a unit costs about what a one-token expert costs whatever m is.  Units
// are numbered by leading pair in pair order (an expert's parts in k order;
// by cost class first when the grid exceeds the resident workgroups, see
// find_unit) and workgroup z serves unit z, so the workgroups with work are
// the first ones launched whatever the order of the pairs: workgroups are
// dealt to the shader engines of an XCD round robin, and a periodic pattern
// of idle workgroups (pairs sorted by expert, say, with four pairs per
// expert) would otherwise put all the work on one of them.  There are at
// most as many units as valid pairs and at most max_sub per expert, so a
// grid that deep covers them.
constexpr int kLeadExperts = static_cast<int>(sizeof(Shared::tab) / (2 * sizeof(int)));

__device__ __forceinline__ bool pair_valid(const KArgs& a, int q, int& e, int& t) {
  e = pair_expert(a, q);
  t = pair_token(a, q);
  return e >= 0 && e < a.n_experts && t >= 0 && t < a.n_tokens;
}

__device__ __forceinline__ bool pair_valid(const KArgs& a, int q, int& e) {
  int t;
  return pair_valid(a, q, e, t);
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
  const bool parts = a.max_sub > 1;  // else every leading pair is one unit
  // pair counts order the units of one chunk and size an expert's parts
  const bool ordered = a.order && a.n_pairs <= kRows;
  // (one chunk: also to spare a one-pair expert's unit the pair scan)
  const bool counts = parts || a.n_pairs <= kRows;
  for (int e = tid; e < a.n_experts; e += kRows) {
    first[e] = 0x7FFFFFFF;
    if (counts) count[e] = 0;
  }
  if (tid == 0) {
    sh.lead = -1;
    sh.lead_m = 0;
  }
  __syncthreads();
  // this thread's pair of the first chunk (q = tid), kept for the ranking
  int my_e = -1, my_t = 0;
  bool my_valid = false;
  for (int q = tid; q < a.n_pairs; q += kRows) {
    int e, t;
    const bool v = pair_valid(a, q, e, t);
    if (q == tid) {
      my_e = e;
      my_t = t;
      my_valid = v;
    }
    if (v) {
      atomicMin(&first[e], q);
      if (counts) atomicAdd(&count[e], 1);
    }
  }
  __syncthreads();
  if (ordered) {
    // One chunk of pairs, more units than resident workgroups: units are
    // numbered by cost class, the longest
    // first, so that the last workgroups to start are short ones: whole
    // experts with 5+, 3-4, 2, 1 tokens, then the parts of parted experts
    // (each a fraction of its expert's k range).  Within a class, leading
    // pairs in pair order.  A whole expert is one unit (one ballot per
    // class); a parted expert's units (at most kMaxSub = 8) are summed bit by
    // bit over ballots; a wavefront's five class totals are packed 10 bits
    // apiece (at most as many units as pairs, so at most 512).
    const int q = tid;
    const int e = my_e, t = my_t;
    const bool lead = my_valid && first[e] == q;
    const int m = lead ? count[e] : 0;
    const int units = lead ? (parts ? min(m, a.max_sub) : 1) : 0;
    const int cls = units > 1 ? 4 : m >= 5 ? 0 : m >= 3 ? 1 : m == 2 ? 2 : 3;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int nbits = parts ? 4 : 1;
    int lane_before = 0;               // units of earlier lanes of this lane's class
    unsigned long long wave_tot = 0;   // the wavefront's class totals, packed
    // classes 0-3 are whole experts (one unit each): one ballot per class
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const unsigned long long bal = __ballot(cls == c && units > 0);
      if (cls == c) lane_before += __popcll(bal & below);
      wave_tot += static_cast<unsigned long long>(__popcll(bal)) << (10 * c);
    }
    // class 4 (parted experts): the unit counts bit by bit
    for (int b = 0; b < nbits; ++b) {
      const unsigned long long bal = __ballot(cls == 4 && ((units >> b) & 1));
      if (cls == 4) lane_before += __popcll(bal & below) << b;
      wave_tot += static_cast<unsigned long long>(__popcll(bal)) << (40 + b);
    }
    if (lane == 0) sh.ball[wave] = wave_tot;
    __syncthreads();
    unsigned long long before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const unsigned long long sw = sh.ball[w];
      before += (w < wave) ? sw : 0ull;
      total += sw;
    }
    int first_unit = static_cast<int>((before >> (10 * cls)) & 1023u) + lane_before;
    for (int c = 0; c < cls; ++c) first_unit += static_cast<int>((total >> (10 * c)) & 1023u);
    if (units > 0 && z >= first_unit && z < first_unit + units) {
      sh.lead = q;
      sh.sub = z - first_unit;
      sh.nsub = units;
      sh.lead_m = m;
      if (m == 1) {  // the pass of a one-pair expert: this pair alone
        sh.pairs[0] = q;
        for (int k = 0; k < kMT2; ++k) sh.toks[k] = t;
      }
    }
    __syncthreads();  // sh.ball is read above and rewritten by the gather; sh.lead is visible
    return sh.lead;
  }
  // more pairs than one chunk, or all units resident at once: units in
  // leading-pair order
  int base = 0;
  for (int c = 0; c < a.n_pairs && base <= z; c += kRows) {
    const int q = c + tid;
    int e = -1, t = 0;
    const bool lead = q < a.n_pairs && pair_valid(a, q, e, t) && first[e] == q;
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
      const int m = counts ? count[e] : 0;
      sh.lead_m = m;
      if (m == 1) {  // the pass of a one-pair expert: this pair alone
        sh.pairs[0] = q;
        for (int k = 0; k < kMT2; ++k) sh.toks[k] = t;
      }
    }
    base += total;
    __syncthreads();  // sh.wsum is rewritten by the next chunk
  }
  return sh.lead;  // sh.lead, sh.sub, sh.nsub and sh.lead_m are not written again in this launch
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

// kMfma (bf16 activations only): passes of kMfmaMinTokens or more tokens
// run on the matrix cores.  It is a separate kernel because the extra path
// changes the compiler's register assignment and loop versioning of the table
// paths, which then run ~10 % slower; calls expected to have few such passes
// take the variant without it.
template <int kMode, bool kMfma>
__device__ __forceinline__ void gemv_main(const KArgs& a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int z = blockIdx.z;
  const int split = blockIdx.y;
  const int row = blockIdx.x * kRows + tid;
  const bool row_ok = row < a.n;

  // the matrix-core form's bf16 pattern table (made visible by the barriers
  // of the unit search below)
  if (kMfma && threadIdx.x < 32) {
    const uint32_t c = threadIdx.x;
    auto bf = [&](int l) -> uint32_t {
      const int t = code_lane_value(c, l);
      return t == 0 ? 0u : (t > 0 ? 0x3F80u : 0xBF80u);  // bf16 +1, -1
    };
    sh.lut[c] = bf(0) | (bf(1) << 16);
    sh.lut[32 + c] = bf(2) | (bf(3) << 16);
  }
  // an invalid pair gets a row of NaN, whichever workgroup leads below:
  // workgroup z marks pairs z, z + gridDim.z, ... (the grid is no deeper
  // than the units can be)
  if (split == 0 && row_ok) {
    for (int q = z; q < a.n_pairs; q += gridDim.z) {
      const int eq = pair_expert(a, q), tq = pair_token(a, q);
      if (eq < 0 || eq >= a.n_experts || tq < 0 || tq >= a.n_tokens)
        a.y[static_cast<int64_t>(q) * a.n + row] = __builtin_nanf("");
    }
  }
  // this workgroup serves unit z: part `sub` of `nsub` of the expert of leading pair p
  // (uniform; p = -1 if there are fewer units)
  // one pair (a single-expert call): it is the only unit and its expert's
  // only pair, so neither the unit search nor the pair scan is needed
  const bool single = a.n_pairs == 1;
  int p;
  if (single) {
    int e0;
    p = __builtin_amdgcn_readfirstlane(pair_valid(a, 0, e0) ? 0 : -1);
  } else {
    p = __builtin_amdgcn_readfirstlane(a.n_experts <= kLeadExperts ? find_unit(a, sh, z) : leader_if_first(a, sh, z));
  }
  if (p < 0) return;
  const int e = __builtin_amdgcn_readfirstlane(pair_expert(a, p));
  const bool parts = a.max_sub > 1 && !single;
  const int sub = parts ? __builtin_amdgcn_readfirstlane(sh.sub) : 0;
  const int nsub = parts ? __builtin_amdgcn_readfirstlane(sh.nsub) : 1;
  // the unit's expert has one valid pair, p (a single-pair call, or one the
  // search counted): its pass is known without the pair scan
  const bool one = single || (a.n_experts <= kLeadExperts && __builtin_amdgcn_readfirstlane(sh.lead_m) == 1);

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

  // one pass of the pair alone: the search placed it in sh.pairs / sh.toks
  // (published by its last barrier); a single-pair call places it here
  if (single) {
    if (tid == 0) {
      sh.pairs[0] = 0;
      const int t0 = pair_token(a, 0);
      for (int m = 0; m < kMT2; ++m) sh.toks[m] = t0;
    }
    __syncthreads();
  }
  int cursor = p;
  for (;;) {
    if (one) {
      if (cursor != p) break;  // its one pass is done
    } else {
      gather<kMfma ? kMT2 : kMT>(a, sh, e, cursor);
    }
    const int mc = one ? 1 : __builtin_amdgcn_readfirstlane(sh.mc);
    if (mc == 0) break;
    cursor = one ? a.n_pairs : __builtin_amdgcn_readfirstlane(sh.next);
    auto store = [&](const auto& acc) {
      constexpr int kN = sizeof(acc) / sizeof(float);
      if (row_ok) {
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          if (m < mc) {
            const int64_t q = sh.pairs[m];
            if (n_slots == 1) a.y[q * a.n + row] = acc[m];
            else a.partial[(static_cast<int64_t>(slot) * a.n_pairs + q) * a.n + row] = acc[m];
          }
        }
      }
    };
    if (kMfma && mc > kMT) {
      float acc[kMT2];
      run_chunk_mfma<2>(a, sh, wexp, b_begin, b_end, acc);
      store(acc);
    } else {
      float acc[kMT];
      if (kMfma && mc >= kMfmaMinTokens) {
        run_chunk_mfma<1>(a, sh, wexp, b_begin, b_end, acc);
      } else switch (mc) {
        case 1: run_chunk<kMode, 1>(a, sh, wexp, b_begin, b_end, acc); break;
        case 2: run_chunk<kMode, 2>(a, sh, wexp, b_begin, b_end, acc); break;
        case 3:  // pair tables take 3 tokens as 4 (the fourth repeats the third, its sums unused)
          run_chunk<kMode, 4>(a, sh, wexp, b_begin, b_end, acc);
          break;
        default: run_chunk<kMode, 4>(a, sh, wexp, b_begin, b_end, acc); break;
      }
      store(acc);
    }
    // the reduction learns each pair's part count from the first unit of its expert
    if (a.pair_sub && split == 0 && sub == 0 && blockIdx.x == 0 && tid < mc) a.pair_sub[sh.pairs[tid]] = nsub;
    if (!one) __syncthreads();  // sh.pairs is rewritten by the next gather
  }
}

// At most 128 VGPRs (4 waves per SIMD, two workgroups per CU as the LDS
// allows); the fp32-row kernel's pair-table builds need a few bytes of
// spill outside the block loop to stay there.
template <int kMode, bool kMfma>
__global__ __launch_bounds__(kRows, 4) void gemv_kernel(KArgs a) {
  gemv_main<kMode, kMfma>(a);
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

// Compute units of device `dev` (cached per device; 256 if the query fails).
static int cus_of_device(int dev) {
  static std::atomic<int> cache[64];
  if (dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int cus_of_stream(hipStream_t s) {
  int dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess) return 256;
  return cus_of_device(dev);
}

int cus_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  return cus_of_device(dev);
}

// Work of one pass over a block, relative to a one-token pass, measured on
// a full layer with every expert given the same token count: on the tables
// (passes of 1..4 tokens) 1, 1.45, 2.1 and 2.18; in the kernel variant with
// the matrix-core form (passes of 1..8 tokens, 3 and more on the matrix
// cores) 1, 1.19, 1.47, 1.52, 2.03, 2.12, 2.2 (interpolated) and 2.31.  An
// expert with m tokens makes floor(m / P) full passes of P tokens and one
// pass of the rest.
static double block_cost(int m, bool mfma) {
  constexpr double kTab[5] = {0.0, 1.0, 1.45, 2.1, 2.18};
  constexpr double kMat[9] = {0.0, 1.0, 1.19, 1.47, 1.52, 2.03, 2.12, 2.2, 2.31};
  if (mfma) return (m / kMT2) * kMat[kMT2] + kMat[m % kMT2];
  return (m / kMT) * kTab[kMT] + kTab[m % kMT];
}

// The matrix-core variant pays off once experts commonly hold 3 or more of
// the call's tokens; it is taken when there are at least as many pairs as
// experts (bf16 activations only).
static bool use_mfma(const GemvArgs& a) { return a.x_mode == 1 && a.n_pairs >= a.n_experts; }

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
  const bool mfma = use_mfma(a);
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
        const double c = block_cost(m, mfma) * bps;
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
GemvPlan plan_gemv(const GemvArgs& a, int cus) {
  struct Entry {
    int64_t n_pairs, n_experts, n, k;
    int cus, x_mode, splits, bps, sub;
  };
  thread_local Entry cache[16];
  thread_local int cache_used = 0, cache_next = 0;
  if (cus <= 0) cus = 256;
  const int nb = static_cast<int>(a.k / kQK);
  const bool parts_ok = a.n_experts <= kLeadExperts;
  int best_splits = 0, best_bps = 0, best_sub = 0;
  for (int i = 0; i < cache_used; ++i) {
    const Entry& c = cache[i];
    if (c.n_pairs == a.n_pairs && c.n_experts == a.n_experts && c.n == a.n && c.k == a.k && c.cus == cus &&
        c.x_mode == a.x_mode) {
      best_splits = c.splits;
      best_bps = c.bps;
      best_sub = c.sub;
      break;
    }
  }
  if (best_splits == 0) {
    estimate_plan(a, cus, best_splits, best_bps, best_sub);
    cache[cache_next] = Entry{a.n_pairs, a.n_experts, a.n, a.k, cus, a.x_mode, best_splits, best_bps, best_sub};
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
  pl.mfma = use_mfma(a);
  // order matters only when not every workgroup of the grid is resident at once
  const int64_t ntiles = (a.n + kRows - 1) / kRows;
  pl.order_units = a.n_pairs * ntiles * best_splits > 2ll * cus;
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
  a.order = pl.order_units ? 1 : 0;
  const int ntiles = static_cast<int>((ga.n + kRows - 1) / kRows);
  // units: at most one per valid pair, and with the leader table at most
  // max_sub per expert; beyond it workgroup z serves pair z
  const int64_t units = a.n_experts <= kLeadExperts
                            ? std::min<int64_t>(a.n_pairs, static_cast<int64_t>(a.n_experts) * pl.max_sub)
                            : a.n_pairs;
  const dim3 grid(ntiles, pl.splits, static_cast<unsigned>(units));
  switch (ga.x_mode) {
    case kXBF16:
      if (pl.mfma) hipLaunchKernelGGL((gemv_kernel<kXBF16, true>), grid, dim3(kRows), 0, s, a);
      else hipLaunchKernelGGL((gemv_kernel<kXBF16, false>), grid, dim3(kRows), 0, s, a);
      break;
    default: hipLaunchKernelGGL((gemv_kernel<kXF32, false>), grid, dim3(kRows), 0, s, a); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.partial_bytes == 0 || !reduce) return err;
  const dim3 grid2(static_cast<unsigned>((ga.n + 255) / 256), static_cast<unsigned>(ga.n_pairs));
  hipLaunchKernelGGL(reduce_splits_kernel, grid2, dim3(256), 0, s, a.partial, pl.splits, pl.splits * pl.max_sub,
                     a.pair_sub, a.n_pairs, a.pe, a.pt, a.ppt, a.n_experts, a.n_tokens, a.n, a.y);
  return hipGetLastError();
}

}  // namespace stq
