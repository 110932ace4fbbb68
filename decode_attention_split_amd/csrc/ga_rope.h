// ga_rope.h -- the rotary embedding of one row element, shared by the RoPE + append kernel
// and the decode that fuses it (so both give the same bits).
//
// Rotate-half pairs (i, i + D/2) of a D-element head: pair i turns by the angle
// p * base^(-2i/D) when i < R/2 (R = rotary_dim, the rotated width) and every other
// element passes through; computed in fp64 from the bf16 inputs and rounded once to bf16
// ("Gemma support" pull request, Summary: RoPE with its own base per layer type, and
// proportional RoPE; "Gemma 4 12B (unified multimodal)" record, CONTEXT_SCALING_METHOD:
// rope_type default on sliding layers (R = D), proportional on full layers (R < D, the
// frequencies still over the whole head); "Gemma4-26B-A4B on Apple Silicon ... (NO-GO)",
// Results, Break 4: partial rotary on the low portion of full-attention heads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

// double -> bf16 bits, nearest with ties to even, in one rounding
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  const double f = frexp(fabs(x), &e);     // |x| = f 2^e, f in [0.5, 1)
  const double m = rint(ldexp(f, 8));       // 8 significant bits (128..256), ties to even
  const float r = (float)ldexp(m, e - 8);   // exact
  return (uint16_t)((__float_as_uint(r) >> 16) | (signbit(x) ? 0x8000u : 0u));
}

// cos and sin of the angle p * base^(-2i/D) of rotate-half pair i of a D-element head.
__device__ __forceinline__ void rope_angle(int i, int D, double base, long long p, double* cs,
                                           double* sn) {
  const double ang = (double)p * pow(base, -2.0 * i / D);
  sincos(ang, sn, cs);
}

__device__ __forceinline__ double bf16_to_f64(uint16_t x) {
  return (double)__uint_as_float((uint32_t)x << 16);
}

// A rotated pair (x0, x1) = (x_i, x_{i+D/2}): first -> x0 cos - x1 sin, second ->
// x1 cos + x0 sin.
__device__ __forceinline__ uint16_t rope_first(uint16_t x0, uint16_t x1, double cs, double sn) {
  return f64_to_bf16(bf16_to_f64(x0) * cs - bf16_to_f64(x1) * sn);
}
__device__ __forceinline__ uint16_t rope_second(uint16_t x0, uint16_t x1, double cs, double sn) {
  return f64_to_bf16(bf16_to_f64(x1) * cs + bf16_to_f64(x0) * sn);
}

// Element d of row (D bf16 values) after the rotation at position p with rotated width R
// (the pairs i >= R/2 pass through).
__device__ __forceinline__ uint16_t rope_element(const uint16_t* row, int d, int D, int R,
                                                 double base, long long p) {
  const int H = D / 2;
  const int i = d < H ? d : d - H;
  if (2 * i >= R) return row[d];
  double cs, sn;
  rope_angle(i, D, base, p, &cs, &sn);
  return d < H ? rope_first(row[i], row[i + H], cs, sn) : rope_second(row[i], row[i + H], cs, sn);
}

}  // namespace ga
