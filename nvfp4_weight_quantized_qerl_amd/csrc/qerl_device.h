// Device-side helpers shared by the HIP kernels of libqerl (gfx950 only).
//
// Number formats (the pages fix E2M1 codes with one E4M3 scale per 16
// elements and one FP32 scale per tensor [QeRL summary, §3.4, Eq. 6]):
//   E2M1   sign bit 3, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7
//   E4M3   OCP FP8 E4M3FN, bias 7, largest finite 448
//   bf16   upper half of an fp32
//
// Hardware facts relied on (gfx950, checked on the device by the parity
// tests of the kernels that use them):
//   v_cvt_scalef32_pk_f32_fp4  two E2M1 codes of one byte -> two fp32,
//                              low nibble first; only the power-of-two part
//                              of the scale operand is applied
//   v_cvt_f32_fp8              decodes OCP E4M3FN
//   v_cvt_pk_bf16_f32          two fp32 -> packed bf16, round to nearest even
//   v_mfma_f32_32x32x16_bf16   A[i][k]: lane l holds i = l%32,
//                              k = 8*(l/32) + 0..7; B[k][j]: j = l%32, same k;
//                              D[i][j]: lane l, element v holds j = l%32,
//                              i = 8*(v/4) + 4*(l/32) + v%4
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qerl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// OCP E4M3FN byte -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Eight E2M1 codes (one dword, code i in nibble i) times an E4M3 block
// scale -> eight bf16 values (code i in half i of the result), exact:
// e2m1 * s_b has at most 6 significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ uint4 dequant8_bf16(uint32_t codes, float sb) {
  f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  uint4 r;
  r.x = pack_bf16x2(v0[0] * sb, v0[1] * sb);
  r.y = pack_bf16x2(v1[0] * sb, v1[1] * sb);
  r.z = pack_bf16x2(v2[0] * sb, v2[1] * sb);
  r.w = pack_bf16x2(v3[0] * sb, v3[1] * sb);
  return r;
}

// The same for a power-of-two scale sb: v_cvt_scalef32_pk_bf16_fp4 applies
// the power-of-two part of its scale operand, which is all of sb, so each
// instruction gives two exact bf16 products (byte i holds codes 2i, 2i+1).
__device__ __forceinline__ uint4 dequant8_bf16_pow2(uint32_t codes, float sb) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sb, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sb, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sb, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sb, 3));
  return r;
}

__device__ __forceinline__ f32x16_t mfma_bf16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Row of the 32x32 MFMA accumulator held in element v of lane l.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

}  // namespace qerl
