// ga_internal.h -- host-side interfaces between the C ABI (api.hip) and the kernel
// translation units of libgemma_attn.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemma_attn.h"

namespace ga {

// Everything a split-decode launch needs; plain values and device pointers.
struct DecodeArgs {
  const uint16_t* q;      // [B, Hq, D]
  const uint16_t* k;      // [B, Hkv, cap, D]
  const uint16_t* v;      // same, or == k when K = V
  const int32_t* ctx;     // [B]
  const int32_t* q_pos;   // [B]
  float* out;             // [B, Hq, D]
  float* part_acc;        // [B, Hq, S, D]   (unused when S == 1)
  float* part_ml;         // [B, Hq, S, 2]   (m in log2 units, l)
  int B, Hq, Hkv, D, cap, kind, window;
  float scale;            // query scale on the fp32 dot product
  float softcap;          // > 0: on
  float inv_softcap;
  int split_keys;         // keys per split (Ts)
  int n_split;            // S, splits per row (host upper bound)
  int max_keys;           // rows longer than this keep their newest keys
  int* plan;              // matrix-core path: per-unit key prefix sums [B * Hkv + 1]
  int n_blocks;           // matrix-core path: work-groups of the decode launch
};

// Matrix-core path limits: units (batch rows x KV heads) per call, and the fixed grid
// (one work-group of 4 waves per CU of an MI355X).
constexpr int kMfmaMaxUnits = 1024;
constexpr int kMfmaBlocks = 256;

// Split kernels.  Each launch covers B * Hkv * S work-groups; with S == 1 the split
// kernel writes `out` directly, otherwise it writes partials for merge_launch.
hipError_t decode_valu_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream);
int decode_valu_keys_per_iter(int D, int G);   // split_keys must be a multiple of this
bool decode_valu_supported(int D, int G);

// Matrix-core path (head_dim 512, G = 16, K = V): decode plus its unit merge.
hipError_t decode_mfma_launch(const DecodeArgs& a, hipStream_t stream);
bool decode_mfma_supported(int D, int G, bool k_eq_v);
size_t decode_mfma_workspace_bytes(int B, int Hkv);  // partials + plan

hipError_t merge_launch(const DecodeArgs& a, hipStream_t stream);

hipError_t append_launch(int B, int Hkv, int D, int cap, int kind, uint16_t* k_cache,
                         uint16_t* v_cache, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* pos, hipStream_t stream);

hipError_t validate_launch(int B, int cap, int kind, int window, int max_ctx, const int32_t* ctx,
                           const int32_t* q_pos, int32_t* flags, hipStream_t stream);
hipError_t ranges_launch(int B, int cap, int kind, int window, int max_keys, const int32_t* ctx,
                         const int32_t* q_pos, int32_t* out, hipStream_t stream);

}  // namespace ga
