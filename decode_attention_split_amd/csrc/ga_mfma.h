// ga_mfma.h -- matrix-core helpers shared by the MFMA decode kernels (gfx950).
//
// Lane layouts (wave64, l16 = lane % 16, lg = lane / 16), verified on the GPU:
//   v_mfma_f32_16x16x32_bf16  A[m][k]: lane holds m = l16, k = 8 lg + 0..7;
//                             B[k][n]: lane holds n = l16, k = 8 lg + 0..7;
//                             C[m][n]: lane holds n = l16, m = 4 lg + 0..3.
//   ds_read_b64_tr_b16        within a 16-lane block, lane i receives element i of each of
//                             the four 8-byte rows read by lanes 4e..4e+3 (a 4x16 -> 16x4
//                             transpose of bf16 values).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ga_device.h"

namespace ga {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // RNE
}

__device__ __forceinline__ floatx4_t mfma_k32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ floatx4_t mfma_k32(u32x4_t a, u32x4_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Eight e4m3 codes (code i in byte i of w0, w1) -> eight bf16 values, exactly: every
// e4m3 value (3 mantissa bits, exponents 2^-9 .. 2^8) is a bf16 value.  One
// v_cvt_scalef32_pk_bf16_fp8 (scale 1) widens two codes; checked on the GPU to give the
// same bits as v_cvt_pk_f32_fp8 followed by taking each float's upper half, for all 256
// codes in both halves of a word.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// Two 4 x 16-bit operand halves -> one 8 x 16-bit operand (lo in k slots 0..3).
__device__ __forceinline__ uint4 cat4(short4_t lo, short4_t hi) {
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// LDS exchange inside one wave: the hardware keeps a wave's LDS accesses in order; the
// wave-scope fences keep the compiler from moving LDS accesses across this point, so
// lanes may read what other lanes of the same wave wrote before it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ga
