// Device helpers shared by the gfx950 DSA kernels: vector types, MFMA
// wrappers, bf16 rounding and wave64 lane utilities.
//
// MFMA register layouts used throughout (checked on gfx950 with an in-bounds
// probe; lane l of the 64-lane wave):
//   16x16xK:  A operand row   m = l % 16, K-chunk (l / 16)
//             B operand col   n = l % 16, K-chunk (l / 16)
//             C/D element j   row 4*(l/16) + j, col l % 16          (j < 4)
//   32x32xK:  A row m = l % 32, B col n = l % 32, K-chunk (l / 32)
//             C/D element j   row 8*(j/4) + 4*(l/32) + j%4, col l % 32 (j < 16)
// A K-chunk is the lane's contiguous run of K elements (32 fp8 bytes for the
// f8f6f4 forms, 8 bf16 values for the bf16 forms).  A and B use the same
// chunk order, so any consistent permutation of K inside a chunk set is
// harmless to the product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

#define DSA_LDS __attribute__((address_space(3)))

// 16x16x128 FP8 (e4m3fn x e4m3fn) -> fp32, no block scaling.
__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32x32x16 bf16 -> fp32.
__device__ __forceinline__ v16f mfma_32x32x16_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 -> fp32.
__device__ __forceinline__ v4f mfma_16x16x32_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Swap the upper 32 lanes of `a` with the lower 32 lanes of `b` and return
// the pair.  Used for reduce-scatter: for lanes < 32, r.x + r.y = a[l] + a[l+32];
// for lanes >= 32, r.x + r.y = b[l-32] + b[l].
__device__ __forceinline__ float reduce_scatter32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same between 16-lane rows (0,1) and (2,3): row 0/2 lanes get a_row0 + a_row1
// (resp. rows 2,3), row 1/3 lanes get b_row0 + b_row1.
__device__ __forceinline__ float reduce_scatter16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_across_halves(float a) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_across_rows(float a) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_rows(float a) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sum_across_halves(float a) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS round
// trip): Hillis-Steele steps 1, 2, 4, 8 inside each 16-lane row (row_shr;
// lanes whose source falls outside the row read the identity), then lane 15
// of rows 0 and 2 is added into rows 1 and 3 (row_bcast:15) and lane 31 into
// rows 2 and 3 (row_bcast:31).  Op: 0 sum, 1 bitwise or, 2 bitwise and.
template <int Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
  constexpr int id = Op == 2 ? -1 : 0;
  auto f = [](uint32_t a, uint32_t b) { return Op == 0 ? a + b : (Op == 1 ? (a | b) : (a & b)); };
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

// The scan's value in lane 63: the whole wave's sum / or / and (uniform).
template <int Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan<Op>(v), 63);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T clampv(T x, T lo, T hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace dsa
