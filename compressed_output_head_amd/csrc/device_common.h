// Device helpers shared by the gfx950 kernels: operand types, exact integer
// unpacking into fp16 MFMA operands, and number conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace archead {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

// Kernel k-order inside one 8-column run of an MFMA operand.  Operand slot j
// (0..7) of a lane carries column k_order_h(j) of the run for H and the
// residual codes, and column k_order_z(j) for the pre-projection and the A
// codes.  Both operands of every MFMA use the same order, so the dot product
// is unchanged.
//   residual dword bytes (k0k1)(k2k3)(k4k5)(k6k7) unpack to slots k0 k4 k1 k5 k2 k6 k3 k7
//   A-code dwords (j0 j1 j2 j3)(j4 j5 j6 j7) unpack to slots j0 j2 j1 j3 j4 j6 j5 j7
__host__ __device__ constexpr int k_order_h(int j) { return (j >> 1) + 4 * (j & 1); }
__host__ __device__ constexpr int k_order_z(int j) {
  return 4 * (j >> 2) + ((j & 3) >> 1) + 2 * (j & 1);
}

__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 bits_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// 0x6400 is fp16 1024.0, whose ulp is 1: placing an unsigned value u < 1024
// in the low mantissa bits gives exactly 1024 + u; placing a nibble u in bits
// 4..7 gives exactly 1024 + 16u.
constexpr uint32_t kF16Magic2 = 0x64006400u;

// Two pairs of nibbles of one dword as fp16 pairs: lo nibbles of bytes 0 and 2
// give (1024 + u0, 1024 + u2'), hi nibbles give (1024 + 16 u1, 1024 + 16 u3'),
// where u = code + 8 (the XOR with 8 per nibble maps two's complement [-8, 7]
// to offset binary).  Each expression compiles to one v_bitop3_b32.
__device__ __forceinline__ uint32_t nib_lo_pair(uint32_t w) {
  return ((w ^ 0x00080008u) & 0x000F000Fu) | kF16Magic2;
}
__device__ __forceinline__ uint32_t nib_hi_pair(uint32_t w) {
  return ((w ^ 0x00800080u) & 0x00F000F0u) | kF16Magic2;
}

// Eight signed INT4 codes (one dword, low nibble first) -> eight exact fp16
// values in k_order_h:  lo pairs: (1024 + u) - 1032 = q;  hi pairs:
// (1024 + 16u) / 16 - 72 = q (both exact in fp16).
__device__ __forceinline__ h8 unpack_q4(uint32_t w) {
  const h2 lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  const uint32_t r0 = h2_bits(bits_h2(nib_lo_pair(w)) + lo_bias);
  const uint32_t r1 = h2_bits(__builtin_elementwise_fma(bits_h2(nib_hi_pair(w)), sixteenth, hi_bias));
  const uint32_t r2 = h2_bits(bits_h2(nib_lo_pair(w8)) + lo_bias);
  const uint32_t r3 = h2_bits(__builtin_elementwise_fma(bits_h2(nib_hi_pair(w8)), sixteenth, hi_bias));
  const u4 v = {r0, r1, r2, r3};
  return __builtin_bit_cast(h8, v);
}

// Same, each code multiplied by the group code c (exact: |q*c| <= 2040 < 2048).
__device__ __forceinline__ h8 unpack_q4_scaled(uint32_t w, _Float16 c) {
  const h8 q = unpack_q4(w);
  const h8 cc = {c, c, c, c, c, c, c, c};
  return q * cc;
}

// Eight INT8 codes (two dwords) -> eight exact fp16 values in k_order_z.
// The XOR gives u = q + 128 in [0, 255]; 1024 + u - 1152 = q.
__device__ __forceinline__ h8 unpack_i8x8(uint32_t lo, uint32_t hi) {
  const uint32_t x0 = lo ^ 0x80808080u, x1 = hi ^ 0x80808080u;
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t r0 = h2_bits(bits_h2((x0 & 0x00FF00FFu) | kF16Magic2) - bias);
  const uint32_t r1 = h2_bits(bits_h2(((x0 >> 8) & 0x00FF00FFu) | kF16Magic2) - bias);
  const uint32_t r2 = h2_bits(bits_h2((x1 & 0x00FF00FFu) | kF16Magic2) - bias);
  const uint32_t r3 = h2_bits(bits_h2(((x1 >> 8) & 0x00FF00FFu) | kF16Magic2) - bias);
  const u4 v = {r0, r1, r2, r3};
  return __builtin_bit_cast(h8, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four fp32 values as bf16 (round to nearest even, NaN stays NaN), packed in
// order into two dwords (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u2 pack_bf16x4(float a, float b, float c, float d) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 lo = {(__bf16)a, (__bf16)b}, hi = {(__bf16)c, (__bf16)d};
  return u2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Power-of-two exponent S that brings the largest magnitude m of a row into
// [2^14, 2^15) (fp16 keeps every bf16 value of the row above 2^-17 * 2^(-S)
// exact).  Rows that are all zero or not finite get S = 0.
__device__ __forceinline__ int row_exponent(float maxabs) {
  if (!(maxabs > 0.0f) || !(maxabs < __builtin_huge_valf())) return 0;
  int e;
  (void)frexpf(maxabs, &e);  // maxabs = m * 2^e, m in [0.5, 1)
  return 15 - e;
}

// Buffer resource over [base, base + bytes): loads past the end return zero.
// The size is made wave-uniform explicitly: a resource the compiler believes
// divergent is used through a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16 x 16 x 32: lane l holds A row l%16 / B column l%16, k 8*(l/16) .. +8;
// result lane l holds rows 4*(l/16) + e, column l%16.
__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 32 x 32 x 16: lane l holds A row l%32 / B column l%32, k 8*(l/32) .. +8;
// result element v of lane l is row 8*(v/4) + 4*(l/32) + v%4, column l%32.
__device__ __forceinline__ f16x mfma32(h8 a, h8 b, f16x c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

}  // namespace archead
