// Device-side helpers shared by the gfx950 kernels of the paged-attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per KV-cache block

// 16x16 output tile, fp32 accumulate; A[16 x 32] and B[32 x 16] bf16. Lane l
// holds A row l%16 and B column l%16, eight k values each; C rows 4*(l/16)+r,
// column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same tile with k = 16: lane l holds A[l%16][4*(l/16)+r] and B[4*(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// {packed bf16 hi parts, packed bf16 residuals} of two floats: x ~= hi + lo
// to about 2^-17 relative, so a PV product run as two bf16 MFMAs keeps the
// weights' precision.
__device__ __forceinline__ u32x2 split_pack_bf16x2(float a, float b) {
  const uint32_t hi = pack_bf16x2(a, b);
  const float ha = __uint_as_float(hi << 16);
  const float hb = __uint_as_float(hi & 0xffff0000u);
  return u32x2{hi, pack_bf16x2(a - ha, b - hb)};
}

// Fourth word of a raw buffer resource on gfx9-family chips: 32-bit data
// format, so buffer loads move raw bytes.
constexpr int kBufferWordFlags = 0x00020000;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950 LDS transpose read. Within each 16-lane block, lane i receives
// element e = the 16-bit value at offset (i % 4) of the 8 bytes addressed by
// lane 4*e + i/4 of the same block. With lane k addressing row (r0 + k/4),
// columns c0 + 4*(k%4) .. +3 of a row-major matrix, lane i gets the column
// c0 + i of rows r0 .. r0+3: a 4 x 16 tile transposed into MFMA k-order.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Values of lane l and lane l ^ 16 (v_permlane16_swap) or l ^ 32
// (v_permlane32_swap): both results of the swap, in either order.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Reductions across the four 16-lane groups of a wave (lanes that differ in
// bits 4 and 5 of the lane id), on the VALU.
__device__ __forceinline__ float max_across_groups(float v) {
  float a, b;
  pair16(v, a, b);
  v = fmaxf(a, b);
  pair32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_across_groups(float v) {
  float a, b;
  pair16(v, a, b);
  v = a + b;
  pair32(v, a, b);
  return a + b;
}

// Orders this wave's LDS writes before its later LDS reads (and the reverse)
// without a workgroup barrier: LDS instructions of one wave execute in order,
// so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
