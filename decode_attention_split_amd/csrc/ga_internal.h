// ga_internal.h -- host-side interfaces between the C ABI (api.hip) and the kernel
// translation units of libgemma_attn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ga_device.h"
#include "gemma_attn.h"

namespace ga {

// Everything a split-decode launch needs; plain values and device pointers.
struct DecodeArgs {
  const uint16_t* q;      // [B, Hq, D]  (multi-token: [B, T, Hq, D])
  const uint16_t* k;      // [B, Hkv, cap, D]
  const uint16_t* v;      // same, or == k when K = V
  const int32_t* ctx;     // [B]
  const int32_t* q_pos;   // [B]  (multi-token: position of token 0; token t at + t)
  float* out;             // [B, Hq, D]  (multi-token: [B, T, Hq, D])
  float* part_acc;        // [rows, S, D]   (unused when S == 1; rows = B * T * Hq)
  float* part_ml;         // [rows, S, 2]   (m in log2 units, l)
  int B, Hq, Hkv, D, cap, kind, window;
  float scale;            // query scale on the fp32 dot product
  float softcap;          // > 0: on
  float inv_softcap;
  int split_keys;         // keys per split (Ts)
  int n_split;            // S, splits per row (host upper bound)
  int max_keys;           // rows longer than this keep their newest keys
  int* plan;              // matrix-core path: per-unit work-group prefix sums [B * Hkv + 1]
  int n_blocks;           // matrix-core path: work-groups that cover the chip (its CUs)
  int launch_rows = 0;    // matrix-core path: batch rows per launch (0: kMfmaMaxUnits / Hkv)
  // Fused cache append (gemma_attn_decode_append); new_pos == nullptr: none.
  const uint16_t* k_new;  // [B, Hkv, D]
  const uint16_t* v_new;  // [B, Hkv, D], or nullptr for K = V
  const int32_t* new_pos; // [B] absolute position of the appended token
  uint16_t* k_dst;        // == k, writable
  uint16_t* v_dst;        // == v, writable (nullptr for K = V)
  int deterministic;      // vector path: fixed step order (bit-reproducible sums)
  // Rotary embedding fused with the append (vector path, one token): q and the new K row
  // rotate at new_pos[b] inside the decode; the rotated q also goes to q_rot_out.
  int rope = 0;
  int rope_dim = 0;
  const double* rope_table = nullptr;  // [B, rope_dim / 2] (cos, sin) pairs
  uint16_t* q_rot_out = nullptr;
  // Multi-token decode: T query tokens per row, handled in chunks of Tc tokens; a unit
  // (b, g, chunk) walks the union of its tokens' key ranges (at most max_union keys).
  int T = 1, Tc = 1, n_chunks = 1;
  int Gh = 1;             // query heads per KV head (Hq / Hkv)
  int max_union = 0;
  // fp8 e4m3 caches (fp8 != 0): codes [B, Hkv, cap, D] and float32 row scales
  // [B, Hkv, cap]; for K = V the V fields equal the K fields.
  int fp8 = 0;
  // fp8 fused append (single token): where the quantized new rows go (codes, scales)
  uint8_t* k8_dst = nullptr;
  float* ks_dst = nullptr;
  uint8_t* v8_dst = nullptr;  // nullptr for K = V
  float* vs_dst = nullptr;
  const uint8_t* k8 = nullptr;
  const uint8_t* v8 = nullptr;
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
};

// Key range a decode unit walks.  One token: that row's range.  Several tokens: the
// union of the ranges of tokens t0 = chunk * Tc .. t1 of batch row b.  Each token's
// range is an interval whose ends never decrease with the position and move by at most
// one per token, so the union of the non-empty ones is one interval.  It lies inside
// the cache's present positions (ring: ctx - W .. ctx - 1), so its slots wrap at most
// once.  Longer than max_union only when preconditions are violated: then it keeps its
// newest keys, as row_range does.
// (unit_range_of: the same from row b's context length and first position, read once by
// a caller that needs them again)
__device__ __forceinline__ RowRange unit_range_of(const DecodeArgs& a, int ctx, int q0,
                                                  int chunk) {
  if (a.T == 1) return row_range(ctx, q0, a.window, a.kind, a.cap, a.max_keys);
  const int t0 = chunk * a.Tc;
  const int t1 = min(a.T, t0 + a.Tc) - 1;
  int lo = 0, hi = -1;
  for (int t = t0; t <= t1; ++t) {
    const RowRange r = row_range(ctx, q0 + t, a.window, a.kind, a.cap, a.max_keys);
    if (r.n <= 0) continue;
    if (hi < lo) lo = r.lo;  // first non-empty token
    hi = r.hi;
  }
  int n = hi - lo + 1;
  if (n < 0) n = 0;
  if (n > a.max_union) {
    lo = hi - a.max_union + 1;
    n = a.max_union;
  }
  RowRange u;
  u.lo = lo;
  u.hi = n > 0 ? hi : lo - 1;
  u.n = n;
  u.slot_lo = n > 0 ? (a.kind == GA_CACHE_RING ? lo % a.cap : lo) : 0;
  return u;
}
__device__ __forceinline__ RowRange unit_range(const DecodeArgs& a, int b, int chunk) {
  return unit_range_of(a, a.ctx[b], a.q_pos[b], chunk);
}

// The slot a token appended at position p goes to (-1: out of range, which the plain
// append skips too).
__device__ __forceinline__ int appended_slot_at(const DecodeArgs& a, int p) {
  if (p < 0 || (a.kind == GA_CACHE_LINEAR && p >= a.cap)) return -1;
  return a.kind == GA_CACHE_RING ? p % a.cap : p;
}
// Fused append: the physical slot the appended token of batch row b goes to, or -1 when
// nothing is appended (no fused append, or a position out of range).
__device__ __forceinline__ int appended_slot(const DecodeArgs& a, int b) {
  return a.new_pos ? appended_slot_at(a, a.new_pos[b]) : -1;
}

// Fused append: moves the new K (and V) row of unit (b, g) into its slot, bit for bit.
// Used by exactly one work-group per unit; threads tid < D / 8 each move 16 bytes.  load()
// issues the reads at the start of the work-group, store() writes at its end, so the
// work-group never waits on them.  No work-group of the same launch reads that slot from
// the cache: every reader of a key whose slot equals the appended slot takes the row from
// k_new / v_new instead, which is what the cache holds after an append, so the launch
// equals append-then-decode.
struct AppendRow {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 k, v;
  size_t dst;
  bool on;
  // The loads are unconditional (from the first 16 bytes of q when this thread moves
  // nothing), so no branch joins around them and nothing waits for them before store().
  __device__ __forceinline__ void load(const DecodeArgs& a, int b, int g, int slot, int tid,
                                       bool mine) {
    const int chunks = a.D / 8;
    on = mine && slot >= 0 && tid < chunks;
    const size_t unit = (size_t)b * a.Hkv + g;
    dst = (unit * a.cap + (on ? slot : 0)) * chunks + tid;
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
    const u32x4* ks = on ? reinterpret_cast<const u32x4*>(a.k_new) + unit * chunks + tid : q;
    const u32x4* vs = on && a.v_dst ? reinterpret_cast<const u32x4*>(a.v_new) + unit * chunks + tid
                                    : ks;
    k = *ks;
    v = *vs;
  }
  // The same loads before the slot is known (place() gives it before store()), so the
  // work-group does not wait for the position at its start.
  __device__ __forceinline__ void load_unplaced(const DecodeArgs& a, int b, int g, int tid,
                                                bool mine) {
    const int chunks = a.D / 8;
    on = mine && a.new_pos != nullptr && tid < chunks;  // (new_pos set: k_new is too)
    const size_t unit = (size_t)b * a.Hkv + g;
    dst = unit;
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
    const u32x4* ks = on ? reinterpret_cast<const u32x4*>(a.k_new) + unit * chunks + tid : q;
    const u32x4* vs = on && a.v_dst ? reinterpret_cast<const u32x4*>(a.v_new) + unit * chunks + tid
                                    : ks;
    k = *ks;
    v = *vs;
  }
  __device__ __forceinline__ void place(const DecodeArgs& a, int slot, int tid) {
    on = on && slot >= 0;
    dst = (dst * a.cap + (on ? slot : 0)) * (a.D / 8) + tid;
  }
  __device__ __forceinline__ void store(const DecodeArgs& a) const {
    if (!on) return;
    reinterpret_cast<u32x4*>(a.k_dst)[dst] = k;
    if (a.v_dst) reinterpret_cast<u32x4*>(a.v_dst)[dst] = v;
  }
};

// Matrix-core path (global K = V geometry): work-groups of kMfmaWaves waves, one per CU
// (the grid follows the device's CU count, at most kMaxBlocks); at most kMfmaMaxUnits
// units (batch rows x KV heads) per launch, larger batches run as several launches.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaMaxUnits = 1024;
constexpr int kMaxBlocks = 256;  // the CU count of an MI355X

// Split kernels.  Each launch covers B * Hkv * S work-groups; with S == 1 the split
// kernel writes `out` directly, otherwise it writes partials for merge_launch.
hipError_t decode_valu_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream);
bool decode_valu_supported(int D, int G);

// Matrix-core path (head_dim 512, G = 16, K = V): decode plus its unit merge.  The grid
// of one launch for `units` units (split_keys 0: balanced over n_blocks work-groups), and
// the workspace of one launch: a partial per work-group plus the plan.
hipError_t decode_mfma_launch(const DecodeArgs& a, hipStream_t stream);
bool decode_mfma_supported(int D, int G, bool k_eq_v);
long long decode_mfma_grid(int units, int n_blocks, int split_keys, int max_keys);
size_t decode_mfma_workspace_bytes(long long grid, int units);

// Matrix-core path for 16 query rows per unit (several tokens x heads of one KV head):
// bf16 caches, head_dim 128 / 256, or 512 with K = V; partials as the vector path's.
hipError_t decode_rows16_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream);
int decode_rows16_waves(int D);  // waves per work-group of the multi-token matrix-core kernel
bool decode_rows16_supported(int D, bool k_eq_v);

hipError_t merge_launch(const DecodeArgs& a, hipStream_t stream);

// Streaming read of `bytes` (a multiple of 1 KiB) over `blocks` work-groups of four waves;
// sink receives blocks * 4 * 64 16-byte values.
hipError_t stream_read_launch(const void* src, size_t bytes, void* sink, int blocks,
                              hipStream_t stream);

// T tokens per row at positions pos[b] + t (T = 1: the single-token append).
hipError_t append_launch(int B, int T, int Hkv, int D, int cap, int kind, uint16_t* k_cache,
                         uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* pos, hipStream_t stream);

// Quantizing append of T tokens per row into fp8 caches (codes + row scales); V
// pointers are nullptr for K = V.
hipError_t append_fp8_launch(int B, int T, int Hkv, int D, int cap, int kind, uint8_t* k_codes,
                             float* k_scales, uint8_t* v_codes, float* v_scales,
                             const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos,
                             hipStream_t stream);

// Rotary embedding of q (-> q_out) and of k_new fused with the append of T tokens per row
// at positions pos[b] + t (v_new appended unrotated; v_cache nullptr for K = V).
hipError_t rope_append_launch(int B, int T, int Hq, int Hkv, int D, int cap, int kind, int R,
                              double base, const uint16_t* q, uint16_t* q_out, uint16_t* k_cache,
                              uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                              const int32_t* pos, const double* table, hipStream_t stream);
// cos / sin of every rotate-half pair at position pos[b]: table [B, R / 2, 2] doubles.
hipError_t rope_table_launch(int B, int R, int D, double base, const int32_t* pos, double* table,
                             hipStream_t stream);

// Flags of the B * T query tokens at positions q_pos[b] + t.
hipError_t validate_launch(int B, int T, int cap, int kind, int window, int max_ctx,
                           const int32_t* ctx, const int32_t* q_pos, int32_t* flags,
                           hipStream_t stream);
hipError_t ranges_launch(int B, int cap, int kind, int window, int max_keys, const int32_t* ctx,
                         const int32_t* q_pos, int32_t* out, hipStream_t stream);

}  // namespace ga
