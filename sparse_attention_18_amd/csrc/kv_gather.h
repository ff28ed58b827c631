// Gather of selected latent KV rows into LDS tiles, shared by the sparse
// attention and the indexer alignment loss (gfx950).
//
// A tile holds kBN = 32 rows of D = 576 bf16 values (latent 512 + rope 64) as
// a sequence of 1 KB blocks, row-block major: block (r / 8) * 9 + c / 8 holds
// 16-byte chunks 8(c/8)..+7 of rows 8(r/8)..+7, and chunk c of row r sits in
// it at slot (r % 8) * 8 + ((c % 8) ^ ((r >> 1) & 7)).  One LDS-DMA load
// (global_load_lds_dwordx4, 64 lanes x 16 B) fills one block, so a wave's
// loads need one row offset per row block and immediate offsets; MFMA operand
// reads of 16 consecutive rows hit 16 distinct bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

constexpr int kD = 576;                      // latent + rope
constexpr int kDL = 512;                     // latent (value) width
constexpr int kBN = 32;                      // keys per tile
constexpr int kChunks = kD * 2 / 16;         // 72 chunks of 16 B per row
constexpr int kPitch = kChunks * 16;         // 1152 B
constexpr int kTileBytes = kBN * kPitch;     // 36864 B
constexpr int kTileInsts = kBN * kChunks / 64;  // 36 wave-wide 1 KB loads per tile
constexpr int kGroups = kChunks / 8;           // 9 chunk groups per row
constexpr int kBlock = 1024;                   // 8 rows x 8 chunks: one DMA load
constexpr int kRowBlockBytes = kGroups * kBlock;   // 8 rows x 72 chunks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(kBN * kChunks % 64 == 0, "tile must be whole 1 KB loads");

__device__ __forceinline__ v8bf as_v8bf(const v4i &x) { return __builtin_bit_cast(v8bf, x); }

// Byte offset, inside a tile, of 16-byte chunk c of row r (see the layout note).
__device__ __forceinline__ int tile_off(int r, int c) {
  return ((r >> 3) * kGroups + (c >> 3)) * kBlock + ((r & 7) * 8 + ((c ^ (r >> 1)) & 7)) * 16;
}

// LDS-DMA loads in scalar-base form: lane i's 16 bytes come from
// base + voff(i) + offset and land at M0 + offset + 16 i.  Four loads share
// one M0 value and fill the consecutive 1 KB blocks M0 + 1024 k (offset
// 1024 k); the instruction offset moves the global address as well, so
// base k is passed already shifted by -1024 k.  The bases are uniform
// (SGPR pairs); the per-lane part is one 32-bit offset.
// A uniform pointer as an SGPR-pair value.  readfirstlane returns a signed
// int: both halves go through uint32_t so that neither is sign-extended.
__device__ __forceinline__ uint64_t sbase(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ void lds_dma16_x4(uint32_t voff, uint64_t b0, uint64_t b1, uint64_t b2,
                                             uint64_t b3, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "global_load_lds_dwordx4 %1, %3 offset:1024\n\t"
      "global_load_lds_dwordx4 %1, %4 offset:2048\n\t"
      "global_load_lds_dwordx4 %1, %5 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(b0), "s"(b1), "s"(b2), "s"(b3), "s"(lds_base)
      : "memory");
}

// Vector-address form (paged caches, whose rows may lie more than 4 GB
// apart): lane i's 16 bytes come from a_k(i) + 1024 k and land at
// M0 + 1024 k + 16 i, so a_k is passed already shifted by -1024 k.
__device__ __forceinline__ void lds_dma16v_x4(uint64_t a0, uint64_t a1, uint64_t a2, uint64_t a3,
                                              uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "global_load_lds_dwordx4 %2, off offset:1024\n\t"
      "global_load_lds_dwordx4 %3, off offset:2048\n\t"
      "global_load_lds_dwordx4 %4, off offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ void lds_dma16v_x1(uint64_t a0, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(a0), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ void lds_dma16_x1(uint32_t voff, uint64_t b0, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(b0), "s"(lds_base)
      : "memory");
}

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace dsa
