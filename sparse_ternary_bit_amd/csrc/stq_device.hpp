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

// One block unpacked into whole words.  Blocks start at even addresses; the
// two cases below are the two possible alignments modulo 4.  Every load is
// 4-byte aligned and stays inside the 4-byte words that hold the block, so
// it never crosses into a page the block does not touch.
struct Block {
  uint32_t d16;
  uint32_t qs[8];
  uint32_t qh[2];
};

__device__ __forceinline__ uint32_t funnel16(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_alignbyte(hi, lo, 2);  // (hi:lo) >> 16
}

// Unpack from 11 consecutive aligned words starting at the word holding the
// block's first byte; `odd` says the block starts at byte 2 of that word.
__device__ __forceinline__ Block block_from_words(const uint32_t (&v)[11], bool odd) {
  Block b;
  if (odd) {
    b.d16 = v[0] >> 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) b.qs[i] = v[i + 1];
    b.qh[0] = v[9];
    b.qh[1] = v[10];
  } else {
    b.d16 = v[0] & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) b.qs[i] = funnel16(v[i + 1], v[i]);
    b.qh[0] = funnel16(v[9], v[8]);
    b.qh[1] = funnel16(v[10], v[9]);
  }
  return b;
}

__device__ __forceinline__ Block load_block_global(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t* w = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
  uint32_t v[11];
#pragma unroll
  for (int i = 0; i < 11; ++i) v[i] = __builtin_nontemporal_load(w + i);
  return block_from_words(v, (a & 2) != 0);
}

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

// Block at byte offset `off` (even) of buffer r.
__device__ __forceinline__ Block load_block_buf(Rsrc r, uint32_t off) {
  const uint32_t base = off & ~3u;
  uint32_t v[11];
#pragma unroll
  for (int i = 0; i < 11; ++i) v[i] = buf_u32(r, base + 4 * i, 0);
  return block_from_words(v, (off & 2u) != 0);
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
