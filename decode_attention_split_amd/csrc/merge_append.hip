// merge_append.hip -- log-sum-exp merge of split partials, cache append, and the two
// debug kernels (precondition flags, key-range dump).  gfx950.
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_quant.h"
#include "ga_rope.h"

namespace ga {
namespace {

// LSE merge ("Gemma support" pull request, Performance: split decode attention).
// Split s of row (b, h) left m_s (log2 units), l_s = sum 2^(s2 - m_s) and
// acc_s = sum 2^(s2 - m_s) v.  With M = max m_s:
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   out = 0 for an empty row.
// One work-group per row; the row's split count comes from the same unit_range the
// split kernel used, so exactly the splits that were written are read.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxSplitsLds = 1024;

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(DecodeArgs a) {
  __shared__ float s_w[kMergeMaxSplitsLds];
  __shared__ float s_red[2][kMergeThreads / 64];
  const size_t bh = blockIdx.x;  // row (b, h), or (b, t, h) with several tokens
  const int b = (int)(bh / ((size_t)a.T * a.Hq));
  const int t = (int)(bh / a.Hq % a.T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.n_split, D = a.D;
  const RowRange r = unit_range(a, b, t / a.Tc);
  const int ns = (r.n + a.split_keys - 1) / a.split_keys;  // <= S
  float* out = a.out + bh * D;
  if (ns == 0) {
    for (int d = tid; d < D; d += kMergeThreads) out[d] = 0.0f;
    return;
  }
  const float* ml = a.part_ml + bh * S * 2;
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kMergeThreads) mloc = fmaxf(mloc, ml[2 * s]);
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
  if (lane == 0) s_red[0][wave] = mloc;
  __syncthreads();
  float M = s_red[0][0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[0][w]);
  // split weights 2^(m_s - M) into LDS, and L = sum_s l_s 2^(m_s - M)
  float lsum = 0.0f;
  // With several tokens a split may hold no key of this row (m = -inf): weight 0; a row
  // with no key at all (M = -inf) gives 0.
  auto split_weight = [&](int s) {
    const float ms = ml[2 * s];
    return ms == -INFINITY ? 0.0f : exp2_fast(ms - M);
  };
  for (int s = tid; s < ns; s += kMergeThreads) {
    const float w = split_weight(s);
    if (s < kMergeMaxSplitsLds) s_w[s] = w;
    lsum += ml[2 * s + 1] * w;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  if (lane == 0) s_red[1][wave] = lsum;
  __syncthreads();
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) Lsum += s_red[1][w];
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  const float* acc = a.part_acc + bh * S * D;
  auto weight = [&](int s) { return s < kMergeMaxSplitsLds ? s_w[s] : split_weight(s); };
  for (int d = tid; d < D; d += kMergeThreads) {
    float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
    int s = 0;
    for (; s + 4 <= ns; s += 4) {  // four independent loads in flight
      o0 = fmaf(weight(s + 0), acc[(size_t)(s + 0) * D + d], o0);
      o1 = fmaf(weight(s + 1), acc[(size_t)(s + 1) * D + d], o1);
      o2 = fmaf(weight(s + 2), acc[(size_t)(s + 2) * D + d], o2);
      o3 = fmaf(weight(s + 3), acc[(size_t)(s + 3) * D + d], o3);
    }
    for (; s < ns; ++s) o0 = fmaf(weight(s), acc[(size_t)s * D + d], o0);
    out[d] = ((o0 + o1) + (o2 + o3)) * inv;
  }
}

// The same merge with one wave per row (four rows per work-group), for rows with few
// splits.  Lane s < ns reads split s's (m_s, l_s) and forms its weight 2^(m_s - M); the
// wave reduces M and L across lanes, and each accumulation step reads the weights back
// from their lanes.  Lane i owns the float4 chunks i, i + 64, ... of the row; eight
// splits' chunks are loaded before any is used, and the first eight of the lane's first
// chunk are requested together with (m_s, l_s), so a row of up to eight splits costs one
// round of loads.
constexpr int kMergeWaveMaxSplits = 64;
constexpr int kMergeWaveBatch = 8;

__global__ void __launch_bounds__(256) merge_wave_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const size_t rows = (size_t)a.B * a.T * a.Hq;
  const size_t bh = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= rows) return;
  const int b = (int)(bh / ((size_t)a.T * a.Hq));
  const int t = (int)(bh / a.Hq % a.T);
  const int S = a.n_split, D4 = a.D / 4;
  const RowRange r = unit_range(a, b, t / a.Tc);
  const int ns = (r.n + a.split_keys - 1) / a.split_keys;  // <= S <= 64
  const float* ml = a.part_ml + bh * S * 2;
  const float4* acc = reinterpret_cast<const float4*>(a.part_acc + bh * S * a.D);
  // the first batch of the lane's first chunk (a split past the row's last is split
  // ns - 1, or 0: in the workspace, never used)
  constexpr int NB = kMergeWaveBatch;
  const int s_last = ns > 0 ? ns - 1 : 0;
  float4 first[NB];
  if (lane < D4) {
#pragma unroll
    for (int j = 0; j < NB; ++j) first[j] = acc[(size_t)min(j, s_last) * D4 + lane];
  }
  float m_s = -INFINITY, l_s = 0.0f;
  if (lane < ns) {
    m_s = ml[2 * lane];
    l_s = ml[2 * lane + 1];
  }
  float M = m_s;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  // a split with no key of this row (m = -inf) weighs 0; so does every split of a row
  // with no key at all (M = -inf), whose output is 0
  const float w_s = m_s == -INFINITY ? 0.0f : exp2_fast(m_s - M);
  float Lsum = l_s * w_s;
  for (int off = 32; off > 0; off >>= 1) Lsum += __shfl_xor(Lsum, off, 64);
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  float4* out = reinterpret_cast<float4*>(a.out + bh * a.D);
  auto weight = [&](int s) {  // s is the same on every lane
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_s),
                                                    __builtin_amdgcn_readfirstlane(s)));
  };
  for (int d = lane; d < D4; d += 64) {
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < ns; s0 += NB) {
      float4 v[NB];
      if (d == lane && s0 == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = first[j];
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = acc[(size_t)min(s0 + j, s_last) * D4 + d];
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (s0 + j < ns) {
          const float w = weight(s0 + j);
          o.x = fmaf(w, v[j].x, o.x);
          o.y = fmaf(w, v[j].y, o.y);
          o.z = fmaf(w, v[j].z, o.z);
          o.w = fmaf(w, v[j].w, o.w);
        }
      }
    }
    out[d] = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// Cache append: one lane per 16-byte chunk of a new row and token; bit-exact copies.  T
// tokens per row sit at positions pos[b] + t; when two tokens of the call land in the same
// ring slot (t + W < T), only the later one writes, so the latest token stays.
__global__ void append_kernel(int B, int T, int Hkv, int D, int cap, int kind, uint4* k_cache,
                              uint4* v_cache, const uint4* k_new, const uint4* v_new,
                              const int32_t* pos) {
  const int chunks = D / 8;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)B * T * Hkv * chunks) return;
  const int c = (int)(i % chunks);
  const long long btg = i / chunks;  // (b * T + t) * Hkv + g
  const int g = (int)(btg % Hkv);
  const long long bt = btg / Hkv;
  const int b = (int)(bt / T), t = (int)(bt % T);
  const long long p = (long long)pos[b] + t;
  if (p < 0 || (kind == GA_CACHE_LINEAR && p >= cap)) return;  // out of range: skipped
  if (kind == GA_CACHE_RING && t + cap < T) return;              // a later token owns it
  const int slot = kind == GA_CACHE_RING ? (int)(p % cap) : (int)p;
  const size_t dst = (((size_t)b * Hkv + g) * cap + slot) * chunks + c;
  const size_t src = (size_t)btg * chunks + c;
  k_cache[dst] = k_new[src];
  if (v_cache) v_cache[dst] = v_new[src];
}

// Quantizing append into fp8 e4m3 caches: one wave per (b, token, KV head), all tokens at
// once; when two tokens of the call land in the same ring slot (t + W < T) only the later
// one writes, so the latest token stays, as with the plain append.  Lane i < D / 8 holds
// 8 consecutive values of the row.  Per row: amax = max |x|, inv = 448 / amax,
// code = round-to-nearest-even e4m3 of clamp(x * inv, +-448), scale = amax / 448, all in
// float32 with correctly rounded division, as the plain definition states.
__device__ __forceinline__ void quantize_store_row(const uint4* src, uint2* dst_codes,
                                                   float* dst_scale, int lane, int chunks) {
  const bool on = lane < chunks;
  const uint4 w = on ? src[lane] : make_uint4(0, 0, 0, 0);
  float scale;
  const uint2 codes = quantize_row_e4m3(w, on, &scale);
  if (on) dst_codes[lane] = codes;
  if (lane == 0) *dst_scale = scale;
}

__global__ void __launch_bounds__(64)
    append_fp8_kernel(int B, int T, int Hkv, int D, int cap, int kind, uint8_t* k_codes,
                      float* k_scales, uint8_t* v_codes, float* v_scales, const uint4* k_new,
                      const uint4* v_new, const int32_t* pos) {
  const int lane = threadIdx.x;
  const int btg = blockIdx.x;  // (b * T + t) * Hkv + g (the launcher keeps it below 2^31)
  const int g = btg % Hkv;
  const int bt = btg / Hkv;
  const int b = bt / T, t = bt % T;
  const long long p = (long long)pos[b] + t;
  if (p < 0 || (kind == GA_CACHE_LINEAR && p >= cap)) return;  // out of range: skipped
  if (kind == GA_CACHE_RING && t + cap < T) return;              // a later token owns it
  const int slot = kind == GA_CACHE_RING ? (int)(p % cap) : (int)p;
  const size_t row = ((size_t)b * Hkv + g) * cap + slot;
  const int chunks = D / 8;
  const size_t src = (size_t)btg * chunks;
  quantize_store_row(k_new + src, reinterpret_cast<uint2*>(k_codes + row * D), k_scales + row,
                     lane, chunks);
  if (v_codes)
    quantize_store_row(v_new + src, reinterpret_cast<uint2*>(v_codes + row * D), v_scales + row,
                       lane, chunks);
}

// Rotary embedding fused with the cache append ("Gemma support" pull request, Summary: own
// RoPE base on sliding layers, proportional RoPE; "Gemma4-26B-A4B on Apple Silicon",
// Results (Break 4) and Ablations / negative controls: partial rotary on the low part of
// the head dimension on full layers).  Rotate-half pairs (i, i + D/2) with i < R/2 turn by
// pos * base^(-2i/D); the rest pass through; double precision, rounded once to bf16
// (nearest, ties to even).  One block of D threads per row (a thread per element):
// q rows -> q_out, k rows -> their cache slot, v rows copied unrotated to theirs (no k / v
// rows without a cache).  Every thread reads its element and its partner before a barrier
// and writes after it, so q_out may alias q.

// One thread per element (blockDim.x = D), one block per row.
__global__ void __launch_bounds__(512)
    rope_append_kernel(int B, int T, int Hq, int Hkv, int D, int cap, int kind, int R,
                       double base, const uint16_t* q, uint16_t* q_out, uint16_t* k_cache,
                       uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                       const int32_t* pos, const double* table) {
  const int d = threadIdx.x;
  const int rows_per_tok = Hq + (k_cache ? Hkv : 0) + (v_cache ? Hkv : 0);
  const long long row = blockIdx.x;  // ((b * T + t) * rows_per_tok + r)
  const int r = (int)(row % rows_per_tok);
  const long long bt = row / rows_per_tok;
  const int b = (int)(bt / T), t = (int)(bt % T);
  const long long p = (long long)pos[b] + t;
  const uint16_t* src;
  uint16_t* dst;
  bool rotate = true;
  if (r < Hq) {
    src = q + (bt * Hq + r) * D;
    dst = q_out + (bt * Hq + r) * D;
  } else {
    const bool is_k = r < Hq + Hkv;
    const int g = is_k ? r - Hq : r - Hq - Hkv;
    // out of range: skipped (as the plain append); on a ring a later token of this call
    // that lands in the same slot (t + W < T) owns it
    if (p < 0 || (kind == GA_CACHE_LINEAR && p >= cap)) return;
    if (kind == GA_CACHE_RING && t + cap < T) return;
    const int slot = kind == GA_CACHE_RING ? (int)(p % cap) : (int)p;
    const uint16_t* nsrc = is_k ? k_new : v_new;
    src = nsrc + (bt * Hkv + g) * D;
    dst = (is_k ? k_cache : v_cache) + (((long long)b * Hkv + g) * cap + slot) * D;
    rotate = is_k;
  }
  uint16_t y;
  const int H = D / 2, i = d < H ? d : d - H;
  if (table && rotate && 2 * i < R) {  // one token (T = 1): the angles of the cos / sin table
    const int n = R / 2;
    const double cs = table[((size_t)b * n + i) * 2], sn = table[((size_t)b * n + i) * 2 + 1];
    y = d < H ? rope_first(src[i], src[i + H], cs, sn) : rope_second(src[i], src[i + H], cs, sn);
  } else {
    y = rope_element(src, d, D, rotate ? R : 0, base, p);
  }
  __syncthreads();  // every element and partner of the row is read before any write
  dst[d] = y;
}

// Thread (b, i): cos and sin of rotate-half pair i (of a D-element head) at position pos[b].
__global__ void __launch_bounds__(256)
    rope_table_kernel(int B, int R, int D, double base, const int32_t* pos, double* table) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = R / 2;
  if (e >= (long long)B * half) return;
  const int b = (int)(e / half), i = (int)(e % half);
  double cs, sn;
  rope_angle(i, D, base, pos[b], &cs, &sn);
  table[2 * e] = cs;
  table[2 * e + 1] = sn;
}

// Precondition flags of every query token (b, t) at position q_pos[b] + t.
__global__ void validate_kernel(int B, int T, int cap, int kind, int window, int max_ctx,
                                const int32_t* ctx_lens, const int32_t* q_pos, int32_t* flags) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)B * T) return;
  const int b = (int)(i / T), t = (int)(i % T);
  const long long ctx = ctx_lens[b], qp = (long long)q_pos[b] + t;
  int f = 0;
  if (ctx < 0 || qp < 0) f |= GA_FLAG_NEGATIVE;
  if (qp >= ctx) f |= GA_FLAG_QPOS_GE_CTX;
  if (kind == GA_CACHE_LINEAR && ctx > cap) f |= GA_FLAG_LINEAR_OVER;
  if (kind == GA_CACHE_RING) {
    long long want_lo = window > 0 ? qp - window + 1 : 0;
    if (want_lo < 0) want_lo = 0;
    if (want_lo < ctx - cap && want_lo <= qp) f |= GA_FLAG_EVICTED;
  }
  if (ctx > max_ctx) f |= GA_FLAG_OVER_MAX_CTX;
  flags[i] = f;
}

__global__ void ranges_kernel(int B, int cap, int kind, int window, int max_keys,
                              const int32_t* ctx_lens, const int32_t* q_pos, int32_t* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const RowRange r = row_range(ctx_lens[b], q_pos[b], window, kind, cap, max_keys);
  out[4 * b + 0] = r.lo;
  out[4 * b + 1] = r.hi;
  out[4 * b + 2] = r.slot_lo;
  out[4 * b + 3] = r.n;
}

}  // namespace

hipError_t merge_launch(const DecodeArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.T * a.Hq;
  if (rows <= 0) return hipSuccess;
  if (a.n_split <= kMergeWaveMaxSplits)
    hipLaunchKernelGGL(merge_wave_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       a);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t append_launch(int B, int T, int Hkv, int D, int cap, int kind, uint16_t* k_cache,
                         uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* pos, hipStream_t stream) {
  const long long n = (long long)B * T * Hkv * (D / 8);
  if (n <= 0 || T <= 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, B, T, Hkv,
                     D, cap, kind, reinterpret_cast<uint4*>(k_cache),
                     reinterpret_cast<uint4*>(v_cache), reinterpret_cast<const uint4*>(k_new),
                     reinterpret_cast<const uint4*>(v_new), pos);
  return hipGetLastError();
}

hipError_t append_fp8_launch(int B, int T, int Hkv, int D, int cap, int kind, uint8_t* k_codes,
                             float* k_scales, uint8_t* v_codes, float* v_scales,
                             const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos,
                             hipStream_t stream) {
  const long long rows = (long long)B * T * Hkv;  // one single-wave work-group each
  if (rows <= 0 || T <= 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_fp8_kernel, dim3((unsigned)rows), dim3(64), 0, stream, B, T, Hkv, D,
                     cap, kind, k_codes, k_scales, v_codes, v_scales,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     pos);
  return hipGetLastError();
}

hipError_t rope_append_launch(int B, int T, int Hq, int Hkv, int D, int cap, int kind, int R,
                              double base, const uint16_t* q, uint16_t* q_out, uint16_t* k_cache,
                              uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                              const int32_t* pos, const double* table, hipStream_t stream) {
  const long long rows = (long long)B * T * (Hq + (k_cache ? Hkv : 0) + (v_cache ? Hkv : 0));
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)rows), dim3(D), 0, stream, B, T, Hq, Hkv,
                     D, cap, kind, R, base, q, q_out, k_cache, v_cache, k_new, v_new, pos,
                     T == 1 ? table : nullptr);
  return hipGetLastError();
}

hipError_t rope_table_launch(int B, int R, int D, double base, const int32_t* pos,
                             double* table, hipStream_t stream) {
  const long long n = (long long)B * (R / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     B, R, D, base, pos, table);
  return hipGetLastError();
}

hipError_t validate_launch(int B, int T, int cap, int kind, int window, int max_ctx,
                           const int32_t* ctx, const int32_t* q_pos, int32_t* flags,
                           hipStream_t stream) {
  const long long n = (long long)B * T;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, B,
                     T, cap, kind, window, max_ctx, ctx, q_pos, flags);
  return hipGetLastError();
}

hipError_t ranges_launch(int B, int cap, int kind, int window, int max_keys, const int32_t* ctx,
                         const int32_t* q_pos, int32_t* out, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(ranges_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, cap, kind,
                     window, max_keys, ctx, q_pos, out);
  return hipGetLastError();
}

}  // namespace ga
