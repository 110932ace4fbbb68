// ga_quant.h -- e4m3 quantization of one cache row with a float32 scale per row, shared by
// the quantizing append kernel and the fp8 decode that appends in its own launch (so both
// store and read the same codes and scale).
//
// Per row: amax = max |x|, inv = 448 / amax, code = round-to-nearest-even e4m3 of
// clamp(x * inv, +-448), scale = amax / 448, in float32 with correctly rounded division
// ("Gemma 4 12B (unified multimodal)" record, KV-cache items (2) and (6): BF16 queries over
// an FP8 KV cache with per-row scales; the per-row absmax scaling is the plain reading).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ga_device.h"

namespace ga {

// One wave quantizes one row of up to 512 values: lane i holds the 8 consecutive values
// 8i .. 8i + 7 in w (bf16 pairs), lanes with on = false hold none (their w is ignored).
// Every lane of the wave must call it (a wave-wide max).  Returns the lane's 8 codes (values
// 0..3 in the bytes of .x, 4..7 in .y) and sets *scale in every lane.
__device__ __forceinline__ uint2 quantize_row_e4m3(const uint4& w, bool on, float* scale) {
  float x[8];
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = on ? bf16_lo(ws[i]) : 0.0f;
    x[2 * i + 1] = on ? bf16_hi(ws[i]) : 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[i] * inv, -448.0f), 448.0f);
  // the second operand of each conversion lands in the higher byte of its pair
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  *scale = amax / 448.0f;
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

}  // namespace ga
