// ga_device.h -- device-side helpers shared by the decode, merge, append and debug
// kernels of libgemma_attn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemma_attn.h"

namespace ga {

constexpr float kLog2e = 1.4426950408889634f;

// Key range one batch row attends to.  The definition (window of exactly `window`
// positions ending at q_pos, the ring holding only the newest W positions, causal
// limit min(q_pos, ctx - 1)) follows the "Gemma 4 12B (unified multimodal)" record's
// statement that a local layer reads exactly w KV entries and its rotating-cache item.
// Every decode kernel, the merge and the debug dump call this one function, so the
// positions selected are identical everywhere.
struct RowRange {
  int lo;       // first valid absolute position
  int hi;       // last valid absolute position
  int slot_lo;  // physical slot of lo
  int n;        // hi - lo + 1, or 0 when empty
};

__device__ __forceinline__ RowRange row_range(int ctx, int q_pos, int window, int kind, int cap,
                                              int max_keys) {
  long long hi = q_pos < ctx - 1 ? q_pos : (long long)ctx - 1;
  if (kind == GA_CACHE_LINEAR && hi > cap - 1) hi = cap - 1;
  long long lo = 0;
  if (window > 0) {
    long long w_lo = (long long)q_pos - window + 1;
    if (w_lo > lo) lo = w_lo;
  }
  if (kind == GA_CACHE_RING) {
    long long r_lo = (long long)ctx - cap;
    if (r_lo > lo) lo = r_lo;
  }
  long long n = hi - lo + 1;
  if (n < 0) n = 0;
  // A row longer than the host bound the split plan was made for keeps its newest keys
  // (never reached when the caller's max_ctx is honoured; validate flags it).
  if (n > max_keys) {
    lo = hi - max_keys + 1;
    n = max_keys;
  }
  RowRange r;
  r.lo = (int)lo;
  r.hi = (int)(n > 0 ? hi : lo - 1);
  r.n = (int)n;
  r.slot_lo = n > 0 ? (kind == GA_CACHE_RING ? (int)(lo % cap) : (int)lo) : 0;
  return r;
}

// Physical slot of the i-th valid key (0 <= i < n): positions are consecutive, so the
// slot advances by one and wraps once at the ring's end (n <= W guarantees no second
// wrap).  For a linear cache slot_lo + i <= hi < C and the wrap never fires.
__device__ __forceinline__ int key_slot(int slot_lo, int i, int cap) {
  const int s = slot_lo + i;
  return s >= cap ? s - cap : s;
}
__device__ __forceinline__ int key_slot(const RowRange& r, int i, int cap) {
  return key_slot(r.slot_lo, i, cap);
}

// bf16 pair held in one dword -> two floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 += a.lo*b.lo + a.hi*b.hi over packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Non-temporal load of streamed cache data (read once per call, not worth keeping in L2
// or the Infinity Cache).  Only for accesses where a lane group reads whole 128-byte lines:
// a line read in halves by separate instructions would be fetched twice.
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(T) == 16)
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p)));
  else
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p)));
}
// Soft-cap c * tanh(x / c), with tanh(y) = 1 - 2 / (exp(2y) + 1): bounded by +-c,
// saturates cleanly (exp -> inf gives 1, exp -> 0 gives -1).  Absolute error of tanh
// is a few float32 ulps of 1.
__device__ __forceinline__ float softcap_tanh(float x, float cap, float inv_cap) {
  float e = exp2_fast(2.0f * kLog2e * x * inv_cap);
  return cap * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
}

// DPP lane permutations inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i inside each 16
constexpr int kDppRowRor8 = 0x128;     // rotate a 16-lane row by 8: lane ^ 8

// The two values of the lane pair {l, l ^ 16} (or {l, l ^ 32}), lower lane first, in both
// lanes of the pair: gfx950's v_permlane16_swap / v_permlane32_swap, all on the VALU.
__device__ __forceinline__ void lane_pair16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false,
                                                  false);
  lo = __int_as_float(r[0]);
  hi = __int_as_float(r[1]);
}
__device__ __forceinline__ void lane_pair32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false,
                                                  false);
  lo = __int_as_float(r[0]);
  hi = __int_as_float(r[1]);
}

// Value held by lane (lane ^ OFF), OFF in {8, 16, 32}, without going through LDS.
template <int OFF>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane offset");
  if constexpr (OFF == 8) {
    return dpp<kDppRowRor8>(v);
  } else {
    float lo, hi;
    if constexpr (OFF == 16) lane_pair16(v, lo, hi); else lane_pair32(v, lo, hi);
    return (lane & OFF) ? lo : hi;
  }
}

// Sum over aligned groups of L lanes; every lane of the group gets the same total.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group size");
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kDppMirror>(x);
  float lo, hi;
  if constexpr (L >= 32) {
    lane_pair16(x, lo, hi);
    x = lo + hi;
  }
  if constexpr (L >= 64) {
    lane_pair32(x, lo, hi);
    x = lo + hi;
  }
  return x;
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48); every
// lane gets the same result.
__device__ __forceinline__ float rows_max(float x) {
  float lo, hi;
  lane_pair16(x, lo, hi);
  x = fmaxf(lo, hi);
  lane_pair32(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float rows_sum(float x) {
  float lo, hi;
  lane_pair16(x, lo, hi);
  x = lo + hi;
  lane_pair32(x, lo, hi);
  return lo + hi;
}

}  // namespace ga
