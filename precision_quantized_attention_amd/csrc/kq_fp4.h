// E2M1 (OCP MX FP4) helpers shared by the quantizers and the SVD-Quant activation pass:
// gfx950's v_cvt_scalef32_pk_fp4_{bf16,f32} divide by 2^(E - 127) (E = the exponent field of the
// float scale operand, 0 .. 254; the mantissa is ignored) and round to the nearest E2M1 value,
// ties to the even code, saturating at +-6 and keeping the sign of zero, and
// v_cvt_scalef32_pk_{bf16,f32}_fp4 multiply back exactly (both directions measured against
// the E2M1 definition on every finite bf16 value and every E).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// running max of the two bf16 magnitudes (15-bit fields) of a dword, packed 16-bit
__device__ __forceinline__ u16x2 mag_max(u16x2 m, uint32_t w) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// 8 values (4 bf16 pairs, or 8 floats) -> one dword of 8 E2M1 codes (byte i from pair i)
__device__ __forceinline__ uint32_t e2m1x8_bf16(const uint32_t* w, float scale) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(v2bf, w[0]), scale, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[1]), scale, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[2]), scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c, __builtin_bit_cast(v2bf, w[3]), scale, 3);
}
__device__ __forceinline__ uint32_t e2m1x8_f32(const float* f, float scale) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], scale, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[2], f[3], scale, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[4], f[5], scale, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[6], f[7], scale, 3);
}
// one dword of 8 E2M1 codes -> 8 values times 2^e: as 4 bf16 pairs, or as 8 floats
__device__ __forceinline__ uint4 e2m1x8_to_bf16(uint32_t c, float scale) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3)));
}
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t c, float scale, float* f) {
  const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 0);
  const v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 1);
  const v2f d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 2);
  const v2f h = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 3);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = d[0]; f[5] = d[1]; f[6] = h[0]; f[7] = h[1];
}

// max of v over the 4 lanes of a quad (lanes 4j .. 4j+3), in every lane of it: two DPP
// quad-permute steps (lane ^ 1, then lane ^ 2)
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
}

// The MX block exponent of a 32-element block from its largest magnitude as float32 bits:
// e = clamp(floor(log2 amax) - 2, -127, 127) (a zero or subnormal amax gives -127), and the
// conversions' scale operand 2^e as the float with exponent field e + 127.
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits) {
  return max((int)(amax_bits >> 23) - 129, -127);
}
__device__ __forceinline__ float mx_scale_operand(int e) {
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

}  // namespace kq
