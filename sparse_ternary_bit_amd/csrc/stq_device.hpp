// Device-side helpers shared by the libstq kernels (gfx950 only).
//
// STQ1_0 block, as this library lays it out (42 bytes, 256 weights):
//   bytes 0..1   fp16 scale d
//   bytes 2..33  eight 32-bit code words; word w carries groups 8w..8w+7, the
//                group with (g & 3) == j in byte lane j, low nibble for
//                groups 8w..8w+3 and high nibble for 8w+4..8w+7
//   bytes 34..41 two 32-bit select words; word h carries groups 32h..32h+31,
//                group g in byte lane (g & 3), bit ((g >> 2) & 7)
// code = nibble | select << 4; zero lane = code >> 3; the other lanes, in
// order, are negative when their bit of (code & 7) is set.  The pages fix the
// group of four with one zero, the 32 patterns in 5 bits, the fp16 scale per
// 256 weights and the 42-byte size (lemmy.durstig.online post 66506,
// "Four weights, five bits"; alphasignal.ai "How STQ1_0 works"); the bit
// order is this library's.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stq {

constexpr int kQK = 256;
constexpr int kBlockBytes = 42;
constexpr int kGroups = 64;
constexpr int kTileRows = 64;

// Packed matrix layout: row tiles of 64 rows (the last tile holds n % 64
// rows when that is nonzero); inside a tile, block 0 of every row in row
// order, then block 1, ...  Block b of a full tile's rows is therefore one
// contiguous, 16-byte aligned run of 64 * 42 = 2688 bytes.
__device__ __forceinline__ int64_t block_offset(int r, int b, int n, int nb) {
  const int t0 = r & ~(kTileRows - 1);
  const int rows = min(kTileRows, n - t0);
  return (static_cast<int64_t>(t0) * nb + static_cast<int64_t>(b) * rows + (r - t0)) * kBlockBytes;
}

// One block unpacked into whole words.
struct Block {
  uint32_t d16;
  uint32_t qs[8];
  uint32_t qh[2];
};

// Raw buffer access: 32-bit byte offsets against a base and a size; a dword
// whose offset is at or past the size reads as 0 (gfx9 buffer range check).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format

// Callers pass workgroup-uniform values; readfirstlane states that to the
// compiler so the descriptor lives in scalar registers (no per-lane loop).
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kRsrcWord3);
}

__device__ __forceinline__ uint32_t buf_u32(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

// The 11 aligned words that cover one 42-byte block.  A block starts at an
// even byte; `off & ~3` is the word holding its first byte, and the three
// loads (16 + 16 + 12 bytes) end at most 2 bytes past the block, inside the
// word holding its last byte.  Inside a tile run the 64 lanes of a wavefront
// loading consecutive blocks cover the run with no gaps.
struct RawBlock {
  uint32_t w[11];
};

__device__ __forceinline__ void load_raw_block(Rsrc r, uint32_t off, RawBlock& raw) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v3i __attribute__((ext_vector_type(3)));
  const int o4 = static_cast<int>(off & ~3u);
  const v4i p0 = __builtin_amdgcn_raw_buffer_load_b128(r, o4, 0, 0);
  const v4i p1 = __builtin_amdgcn_raw_buffer_load_b128(r, o4 + 16, 0, 0);
  const v3i p2 = __builtin_amdgcn_raw_buffer_load_b96(r, o4 + 32, 0, 0);
  raw.w[0] = p0.x; raw.w[1] = p0.y; raw.w[2] = p0.z; raw.w[3] = p0.w;
  raw.w[4] = p1.x; raw.w[5] = p1.y; raw.w[6] = p1.z; raw.w[7] = p1.w;
  raw.w[8] = p2.x; raw.w[9] = p2.y; raw.w[10] = p2.z;
}

// Realign with byte permutes: word i of the block body is bytes 2..5 of
// (w[i+1]:w[i]) when the block starts on a word boundary, and w[i+1] itself
// when it starts 2 bytes into w[0] (`odd`); both are one v_perm with a
// per-thread selector over the same two registers.
__device__ __forceinline__ Block realign_block(const RawBlock& r, bool odd) {
  const uint32_t sel = odd ? 0x07060504u : 0x05040302u;
  const uint32_t seld = odd ? 0x0C0C0302u : 0x0C0C0100u;   // selector byte 0x0C gives 0x00
  Block b;
  b.d16 = __builtin_amdgcn_perm(r.w[1], r.w[0], seld);
#pragma unroll
  for (int i = 0; i < 8; ++i) b.qs[i] = __builtin_amdgcn_perm(r.w[i + 1], r.w[i], sel);
  b.qh[0] = __builtin_amdgcn_perm(r.w[9], r.w[8], sel);
  b.qh[1] = __builtin_amdgcn_perm(r.w[10], r.w[9], sel);
  return b;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Select bit of group (8w + 4u + j) sits at bit 8j + 2(w&3) + u of select word w>>2.
__device__ __forceinline__ uint32_t group_code(const Block& b, int g) {
  const int w = g >> 3, j = g & 3, u = (g >> 2) & 1;
  const uint32_t nib = (b.qs[w] >> (8 * j + 4 * u)) & 15u;
  const uint32_t sel = (b.qh[g >> 5] >> (8 * j + ((g >> 2) & 7))) & 1u;
  return nib | (sel << 4);
}

// Ternary value (-1, 0, +1) of lane `lane` for code c, from the definition.
__device__ __forceinline__ int code_lane_value(uint32_t c, int lane) {
  const int z = static_cast<int>(c >> 3);
  if (lane == z) return 0;
  const int rank = lane - (lane > z ? 1 : 0);
  return ((c >> rank) & 1u) ? -1 : 1;
}

}  // namespace stq
