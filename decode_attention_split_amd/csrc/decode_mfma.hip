// decode_mfma.hip -- matrix-core split-KV decode for the K = V global geometry
// (head_dim 512, 16 query heads per KV head, one cached tensor used as keys and values).
//
// Why matrix cores here: 16 query heads share every key, so a key row of 1 KiB feeds
// 2 * 16 * 512 * 2 = 32 KFLOP (q.k and p.v): 32 flop/byte, above the fp32 vector ridge
// of MI355X (~157 TFLOP/s over 8 TB/s ~ 20 flop/byte), so a VALU kernel cannot reach
// the HBM roofline ("Gemma4-26B-A4B on Apple Silicon", Results, Break 4: 16 query heads
// on one shared K/V head, no separate value projection).
//
// Work partition: the chip gets NB work-groups' worth of keys, C = ceil(T / NB) keys each
// (T = valid keys of the whole batch, rounded to tiles), and every (batch row, KV head)
// unit u with n_u keys gets k_u = ceil(n_u / C) work-groups, each an equal tile-aligned
// share of that unit's keys.  The counts come from prefix sums computed on the device
// from ctx_lens / q_pos, so ragged contexts with few units (one KV head, batch 16-32)
// still spread evenly over every CU -- the failure mode of decode kernels that ignore
// key splitting ("Gemma 4 12B (unified multimodal)" record, item (4): 2 of 132 SMs
// busy) -- and no work-group ever switches units, so its load pipeline never drains.
// Sum k_u <= NB + units, the grid size.  A unit with k_u = 1 is written directly; the
// others leave one partial per work-group (slot = work-group index) for
// merge_units_kernel (log-sum-exp).
//
// One work-group per CU of 8 waves: two groups of 4 waves in lockstep (one barrier per
// step), group h taking the work-group's tiles 4 q + 2 h and 4 q + 2 h + 1, each with its own
// softmax state; the second group's (m, l, acc) join the first's through LDS at the end.
// One work-group per CU (rather than two of 4 waves) keeps a CU's two streams starting
// and ending together: a second work-group on a CU queues behind the first ones' opening
// loads and was measured to finish ~6 us later, leaving its CU half-busy for that time.
// Per group, 16-key tiles taken two per step; wave w of the group owns head_dim slice
// [128 w, 128 w + 128):
//   partial S^T[16 keys][16 heads] = K[16][slice] . Q^T[slice][16] per tile with
//     v_mfma_f32_16x16x32_bf16 (4 per tile): bf16 rows are loaded 16 bytes per lane with
//     each instruction covering whole 128-byte lines of 4 keys (non-temporal), written to
//     the wave's LDS tile and read back as the A operand (key l % 16, d = 128 w + 32 j +
//     8 (l / 16) + 0..7); fp8 codes go straight from registers into the A operand after
//     widening; 4 tiles in flight (8 for fp8); Q^T is held in registers in the same d order;
//   the 4 partials are summed through LDS (one barrier per step of 32 keys), in the same
//     order in every wave, so every wave holds the identical S^T and softmax state;
//   the wave's K = V slice goes once to its own LDS rows (288 B stride) and
//   O^T[slice][16] += V^T[slice][32 keys] . P^T[32 keys][16 heads] with one
//     v_mfma_f32_16x16x32_bf16 per 16-wide d block: the A operand comes from two
//     ds_read_b64_tr_b16 (one per tile; lanes 4e..4e+3 of a 16-lane block read 16
//     consecutive d of key e, lane i then holds the 4 keys at column d0 + i), the B
//     operand is P exactly as the S^T products left it (lane l: head l % 16, keys
//     4 (l / 16) + 0..3 of each tile), split into bf16 hi + lo parts so the probabilities
//     keep ~16 mantissa bits (the bf16 cache data is exact).
// Each wave writes its own slice of the output or partial: no end-of-segment merge.
// The K = V row is read from HBM once and used for both products.  Softmax state per
// head is fp32 in log2 units with lazy rescaling (max raised only past +8).
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_mfma.h"

namespace ga {
namespace {

constexpr int MD = 512;        // head_dim
constexpr int MG = 16;         // query heads per KV head
constexpr int TK = 16;         // keys per tile
constexpr int MNW = 4;         // waves per group, one head_dim slice each
constexpr int MH = kMfmaHalves;  // groups per work-group, in lockstep on alternate key pairs
constexpr int NWV = MNW * MH;  // waves per work-group
constexpr int DQ = MD / MNW;   // head_dim slice of a wave
constexpr int ROWQ = DQ * 2 + 32;   // LDS bytes per key row of a wave's slice (bank spread)
constexpr int WAVE_TILE = TK * ROWQ;
#ifndef GA_FP8_TILES
#define GA_FP8_TILES 8
#endif
#ifndef GA_BF16_TILES
#define GA_BF16_TILES 4
#endif
constexpr float kRescaleLog2 = 8.0f;
// LDS per work-group is sized so that exactly kMfmaBlocksPerCU work-groups fit on a CU
// (160 KiB each): every CU then holds the same number of equal-work work-groups.
constexpr int kLdsCU = 160 * 1024;
constexpr int kLdsOther = 2 * NWV * 2 * 64 * 16 + 3 * (kMfmaMaxUnits + 1) * 4 + 2 * MH * 2 * TK * 4;
constexpr int kLdsTile = kLdsCU / (kMfmaBlocksPerCU + 1) + 1024 - kLdsOther;
constexpr int kLdsKV = 2 * NWV * WAVE_TILE > kLdsTile ? 2 * NWV * WAVE_TILE : kLdsTile;
// the second group's (acc, m, l) go to the first through the second group's tile area
static_assert(2 * WAVE_TILE >= 64 * 8 * 16, "combine area per wave");
static_assert(kLdsKV + kLdsOther <= kLdsCU / kMfmaBlocksPerCU, "LDS budget per work-group");


__device__ __forceinline__ int chunk_keys(int T, int NB) {
  const int per = (T + NB - 1) / NB;
  return T > 0 ? (per + TK - 1) / TK * TK : TK;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then each row adds the last lane of the rows before it (DPP row
// broadcasts), all on the VALU.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return v;
}

template <bool FP8>
__global__ void __launch_bounds__(NWV * 64, kMfmaBlocksPerCU) decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char s_kv[kLdsKV];
  __shared__ floatx4_t s_part[2][MH][MNW][2][64];  // [buffer][group][wave][tile][lane]
  __shared__ __attribute__((aligned(16))) float s_scale[2][MH][2][TK];  // fp8 row scales
  __shared__ float s_ml[MG][2];  // the second group's m and l per head
  __shared__ float s_norm[2][NWV];  // fp8: per-wave largest key scale and |q|
  // Tiles in flight per wave: four bf16 tiles (64 KiB per work-group); fp8 tiles are half
  // the bytes, so eight keep as many bytes in flight (the loop is latency-bound otherwise).
  constexpr int NF = FP8 ? GA_FP8_TILES : GA_BF16_TILES;
  __shared__ int s_n[kMfmaMaxUnits + 1];  // valid keys per unit, then their prefix sums
  __shared__ int s_k[kMfmaMaxUnits + 1];  // work-groups per unit, then their prefix sums
  __shared__ int s_slot[kMfmaMaxUnits];   // slot of each unit's first valid key

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = wave / MNW, wsl = wave % MNW;  // group, and the wave's head_dim slice
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.B * a.Hkv;

  // ---- the partition (every work-group computes it; work-group 0 also publishes it):
  // each unit's key range, then wave 0 alone forms both prefix sums (two barriers).
  for (int u = tid; u < R; u += NWV * 64) {
    const int b = u / a.Hkv;
    const RowRange rr = row_range(a.ctx[b], a.q_pos[b], a.window, a.kind, a.cap, a.max_keys);
    s_n[u + 1] = rr.n;
    s_slot[u] = rr.slot_lo;
  }
  __syncthreads();
  if (wave == 0) {
    int total = 0, nonempty = 0;
    for (int base = 0; base < R; base += 64) {
      const int u = base + lane;
      const int n = u < R ? s_n[u + 1] : 0;
      nonempty += __popcll(__ballot(n > 0));
      const int v = wave_incl_scan(n) + total;
      if (u < R) {
        s_n[u + 1] = v;
        s_k[u + 1] = n;  // kept for the second pass, read back by this lane only
      }
      total = __builtin_amdgcn_readlane(v, 63);
    }
    // k_u = ceil(n_u / C) <= n_u / C + 1, so with C = T / (NB - R') (R' non-empty units)
    // the work-groups with work never exceed NB: all of them are resident at once.
    const int nb_eff =
        a.n_blocks - nonempty >= a.n_blocks / 4 ? a.n_blocks - nonempty : a.n_blocks;
    const int C = chunk_keys(total, nb_eff);
    int groups = 0;
    for (int base = 0; base < R; base += 64) {
      const int u = base + lane;
      const int n = u < R ? s_k[u + 1] : 0;
      const int v = wave_incl_scan((n + C - 1) / C) + groups;
      if (u < R) s_k[u + 1] = v;
      groups = __builtin_amdgcn_readlane(v, 63);
    }
    if (lane == 0) {
      s_n[0] = 0;
      s_k[0] = 0;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int u = tid; u <= R; u += NWV * 64) a.plan[u] = s_k[u];
  // fused append: work-group u (< R <= grid) moves unit u's new row (stored at the end)
  AppendRow app;
  {
    const int u = blockIdx.x < R ? blockIdx.x : 0;
    const int ub = u / a.Hkv;
    app.load(a, ub, u % a.Hkv, appended_slot(a, ub), tid, blockIdx.x < R);
  }
  const int g_id = blockIdx.x;
  if (g_id >= s_k[R]) {
    app.store(a);
    return;
  }
  // unit of this work-group: the u with s_k[u] <= g_id < s_k[u + 1]
  int u, hi_u = R - 1;
  {
    int lo_u = 0;
    while (lo_u < hi_u) {
      const int mid = (lo_u + hi_u) >> 1;
      if (s_k[mid + 1] > g_id) hi_u = mid; else lo_u = mid + 1;
    }
    u = lo_u;
  }
  const int n_u = s_n[u + 1] - s_n[u];
  const int k_u = s_k[u + 1] - s_k[u];
  const int part = g_id - s_k[u];
  const int per = ((n_u + k_u - 1) / k_u + TK - 1) / TK * TK;
  const int seg_lo = part * per;
  const int seg_hi = min(n_u, seg_lo + per);  // non-empty: (k_u - 1) * per < n_u

  const int b = u / a.Hkv, g = u % a.Hkv;
  const int slot_lo = s_slot[u];
  const size_t head0 = (size_t)b * a.Hq + (size_t)g * MG;

  // this wave's two tile buffers (one step's tiles) and its transposed-read addresses
  char* tile_a = s_kv + wave * 2 * WAVE_TILE;
  char* tile_b = tile_a + WAVE_TILE;
  char* lds_ra = tile_a + (4 * lg + (l16 >> 2)) * ROWQ + (l16 & 3) * 8;
  char* lds_rb = tile_b + (4 * lg + (l16 >> 2)) * ROWQ + (l16 & 3) * 8;
  int par = 0;  // s_part double buffer

  // Q^T operand for this wave's slice, in the order the K rows are loaded: head l16,
  // d = 128 w + 32 j + 8 lg + 0..7 (bf16 rows: 16 bytes per lane and j), or
  // d = 128 w + 64 (j / 2) + 16 lg + 8 (j % 2) + 0..7 (fp8 rows: 16 codes per lane and
  // pair of j).  Any order of d works as long as K and Q^T share it.  The fp8 path
  // converts q to fp16 below, once the work-group's range normalization is known.
  uint4 qv[4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (head0 + l16) * MD);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qv[j] = FP8 ? qp[16 * wsl + 8 * (j / 2) + 2 * lg + (j % 2)] : qp[16 * wsl + 4 * j + lg];
  }
  const uint4* kbase = reinterpret_cast<const uint4*>(a.k) + (size_t)u * a.cap * (MD / 8);
  const uint4* cbase = reinterpret_cast<const uint4*>(a.k8) + (size_t)u * a.cap * (MD / 16);
  const float* sbase = FP8 ? a.k_scale + (size_t)u * a.cap : nullptr;
  const int new_slot = appended_slot(a, b);  // fused append: read from k_new instead
  const uint4* knew = a.new_pos ? reinterpret_cast<const uint4*>(a.k_new) + (size_t)u * (MD / 8)
                                : kbase;
  // bf16 loads: lane reads 16 bytes (column lane % 16 of the wave's 256-byte slice) of key
  // lane / 16 + 4 j, so each instruction covers 4 keys x 2 whole 128-byte lines
  const uint4* kbase_l = kbase + 16 * wsl + (lane & 15);
  const uint4* knew_l = knew + 16 * wsl + (lane & 15);

  floatx4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;
  float p_norm = 1.0f, logit_scale = a.scale;  // fp8 range normalization (set below)

  // The work-group's tiles go to the groups in pairs: tiles 4 q, 4 q + 1 to group 0, 4 q + 2,
  // 4 q + 3 to group 1.  Both groups step through group 0's tile count (group 1's extra
  // tiles are past the end: masked, their loads clamped to a valid row).
  const int ntw = (seg_hi - seg_lo + TK - 1) / TK;
  const int nt = MH == 1 ? ntw : 2 * (ntw / 4) + min(ntw % 4, 2);
  auto tile_key0 = [&](int t) {  // first key of this group's local tile t
    return seg_lo + TK * (MH == 1 ? t : 4 * (t >> 1) + 2 * half + (t & 1));
  };

  // One tile's registers: bf16 rows in rg[0..3] (rg[j]: key lane / 16 + 4 j of the tile);
  // fp8 rows: the 32 codes of key l16 in rg[0..1] and that key's scale in rg[2].x.
  auto load = [&](uint4(&rg)[4], int t) {
    if constexpr (FP8) {
      const int key = tile_key0(t) + l16;
      const int kc = key < seg_hi ? key : seg_hi - 1;
      const int slot = key_slot(slot_lo, kc, a.cap);
      const uint4* cp = cbase + (size_t)slot * (MD / 16) + 8 * wsl + lg;
      rg[0] = cp[0];
      rg[1] = cp[4];
      rg[2].x = __float_as_uint(sbase[slot]);  // the scale of this lane's key (l16)
    } else {
      const int key0 = tile_key0(t) + (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + 4 * j;
        const int kc = key < seg_hi ? key : seg_hi - 1;
        const int slot = key_slot(slot_lo, kc, a.cap);
        rg[j] = stream_load(slot == new_slot ? knew_l : kbase_l + (size_t)slot * (MD / 8));
      }
    }
  };

  // One step = two 16-key tiles (ra: keys k0 .. k0 + 15, rb: the next 16): their products
  // and softmax chains interleave, and one barrier and one max update cover 32 keys.
  // Each tile's rows go to the wave's LDS tile in natural d order (the V operand, and for
  // bf16 also the K operand); a tile's S^T partial over this wave's d slice is K rows
  // (A operand) times Q^T.  fp8 codes are widened exactly to fp16 and feed the products
  // from registers.
  auto tile_scores_fp8 = [&](const uint4(&rg)[4], char* tile, floatx4_t& s) {
    s = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const uint4 lo = e4m3x8_to_f16x8(rg[jj].x, rg[jj].y);
      const uint4 hi = e4m3x8_to_f16x8(rg[jj].z, rg[jj].w);
      s = mfma_k32_f16(lo, qv[2 * jj], s);
      s = mfma_k32_f16(hi, qv[2 * jj + 1], s);
      char* w8 = tile + l16 * ROWQ + lg * 32 + jj * 128;  // 16 d per lane and jj
      *reinterpret_cast<uint4*>(w8) = lo;
      *reinterpret_cast<uint4*>(w8 + 16) = hi;
    }
  };
  // bf16: lane writes its 16 bytes of keys lane / 16 + 4 j, then (after the wave's writes)
  // reads the A operand of key l16, d = 32 j + 8 lg + 0..7 of the slice
  auto tile_write_bf16 = [&](const uint4(&rg)[4], char* tile) {
    char* w = tile + (lane >> 4) * ROWQ + (lane & 15) * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(w + 4 * j * ROWQ) = rg[j];
  };

  auto step2 = [&](uint4(&ra)[4], uint4(&rb)[4], int t) {
    const int k0 = tile_key0(t);  // tile b (local t + 1, t even) starts at k0 + TK
    floatx4_t sa, sb;
    if constexpr (FP8) {
      tile_scores_fp8(ra, tile_a, sa);
      tile_scores_fp8(rb, tile_b, sb);
    } else {
      wave_lds_sync();  // the previous step's transposed reads stay before these writes
      tile_write_bf16(ra, tile_a);
      tile_write_bf16(rb, tile_b);
      // the registers are free once written: the next loads go out before the products
      // (unconditional, clamped past the end: keeps the wait counts partial)
      load(ra, t + NF);
      load(rb, t + NF + 1);
      wave_lds_sync();
      sa = floatx4_t{0.f, 0.f, 0.f, 0.f};
      sb = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const char* rda = tile_a + l16 * ROWQ + lg * 16;
      const char* rdb = tile_b + l16 * ROWQ + lg * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sa = mfma_k32(*reinterpret_cast<const uint4*>(rda + 64 * j), qv[j], sa);
        sb = mfma_k32(*reinterpret_cast<const uint4*>(rdb + 64 * j), qv[j], sb);
      }
    }
    s_part[par][half][wsl][0][lane] = sa;
    s_part[par][half][wsl][1][lane] = sb;
    if (FP8 && wsl == 0 && lg == 0) {  // the keys' row scales (times p_norm), for the group
      s_scale[par][half][0][l16] = __uint_as_float(ra[2].x) * p_norm;
      s_scale[par][half][1][l16] = __uint_as_float(rb[2].x) * p_norm;
    }
    if constexpr (FP8) {
      load(ra, t + NF);  // unconditional (clamped past the end): keeps wait counts partial
      load(rb, t + NF + 1);
    }
    __syncthreads();
    float ka[4] = {1.0f, 1.0f, 1.0f, 1.0f}, kb[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (FP8) {  // scales of the keys 4 lg + 0..3 this lane's logits belong to
      const float4 a4 = *reinterpret_cast<const float4*>(&s_scale[par][half][0][4 * lg]);
      const float4 b4 = *reinterpret_cast<const float4*>(&s_scale[par][half][1][4 * lg]);
      ka[0] = a4.x; ka[1] = a4.y; ka[2] = a4.z; ka[3] = a4.w;
      kb[0] = b4.x; kb[1] = b4.y; kb[2] = b4.z; kb[3] = b4.w;
    }
    const floatx4_t fa = ((s_part[par][half][0][0][lane] + s_part[par][half][1][0][lane]) +
                          s_part[par][half][2][0][lane]) + s_part[par][half][3][0][lane];
    const floatx4_t fb = ((s_part[par][half][0][1][lane] + s_part[par][half][1][1][lane]) +
                          s_part[par][half][2][1][lane]) + s_part[par][half][3][1][lane];
    par ^= 1;
    // softmax: lane holds head l16, keys k0 + 4 lg + i (xa) and k0 + 16 + 4 lg + i (xb)
    float xa[4], xb[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float va = fa[i] * ka[i] * logit_scale;  // fp8: the key's row scale
      float vb = fb[i] * kb[i] * logit_scale;
      if (a.softcap > 0.0f) {
        va = softcap_tanh(va, a.softcap, a.inv_softcap);
        vb = softcap_tanh(vb, a.softcap, a.inv_softcap);
      }
      xa[i] = (k0 + 4 * lg + i < seg_hi) ? va * kLog2e : -INFINITY;
      xb[i] = (k0 + TK + 4 * lg + i < seg_hi) ? vb * kLog2e : -INFINITY;
      mx = fmaxf(mx, fmaxf(xa[i], xb[i]));
    }
    mx = rows_max(mx);  // over the 32 keys of the step (four lane rows)
    if (mx > m + kRescaleLog2) {
      const float f = exp2_fast(m - mx);
      l *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= f;
      m = mx;
    }
    // m stays -inf only while every key so far was masked (the second group's steps past
    // the end): then every x is -inf and p must be 0, not exp2(-inf + inf)
    const float mref = m == -INFINITY ? 0.0f : m;
    float pa[4], pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = exp2_fast(xa[i] - mref);
      pb[i] = exp2_fast(xb[i] - mref);
      l += pa[i] + pb[i];
      if constexpr (FP8) {  // K = V: the value row's scale is the key's
        pa[i] *= ka[i];
        pb[i] *= kb[i];
      }
    }
    if constexpr (FP8) {
      // fp16 operands: V^T exact (widened codes), P^T (p * s * p_norm < 2^15) rounded once
      // to 11 significant bits
      const uint4 pf = make_uint4(pack_f16x2(pa[0], pa[1]), pack_f16x2(pa[2], pa[3]),
                                  pack_f16x2(pb[0], pb[1]), pack_f16x2(pb[2], pb[3]));
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const short4_t va =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(lds_ra + db * 32));
        const short4_t vb =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(lds_rb + db * 32));
        acc[db] = mfma_k32_f16(cat4(va, vb), pf, acc[db]);
      }
      return;
    }
    // P^T operands (lane: head l16, keys 4 lg + 0..3), split into bf16 hi + lo parts so
    // the probabilities keep ~16 mantissa bits
    auto split = [](const float(&p)[4], short4_t& ph, short4_t& pl) {
      const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
      const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
      ph = __builtin_bit_cast(short4_t, make_uint2(h01, h23));
      pl = __builtin_bit_cast(short4_t, make_uint2(l01, l23));
    };
    short4_t pah, pal, pbh, pbl;
    split(pa, pah, pal);
    split(pb, pbh, pbl);
    // O^T += V^T P^T over the step's 32 keys with v_mfma_f32_16x16x32_bf16: lane (l16, lg)
    // holds k slots 8 lg + 0..7 = keys 4 lg + 0..3 of tile a, then of tile b, in both
    // operands (the transposed reads give V^T for exactly those keys at column l16, and
    // the softmax left P for exactly those keys), so one product covers both tiles.
    const uint4 ph = cat4(pah, pbh), pl = cat4(pal, pbl);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const short4_t va =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(lds_ra + db * 32));
      const short4_t vb =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(lds_rb + db * 32));
      const uint4 v8 = cat4(va, vb);
      acc[db] = mfma_k32(v8, ph, acc[db]);
      acc[db] = mfma_k32(v8, pl, acc[db]);
    }
  };

  // Straight-line loop body over whole groups of NF tiles (NF / 2 steps); the last tiles
  // run after it, a step's second tile past the end being all masked, so the loop header
  // never sees a path with a buffer's loads still unconsumed (which would make the
  // compiler drain every prefetch there).
  // fp8 computes in fp16 (every e4m3 value is an fp16 value; products accumulate in fp32).
  // Two powers of two per work-group keep the fp16 operands in range: q * q_norm with
  // |q * q_norm| < 2^15, and value weights p * s * p_norm < 2^15 (p <= 2^8 with the lazy
  // rescale, s * p_norm < 2^7 for every key scale s of the work-group's keys).  The logits
  // take 1 / (q_norm p_norm) and the result 1 / p_norm back, both exact.  The key scales'
  // loads go out before the tiles' so that waiting for them leaves the tiles in flight.
  float sk[4];
  if constexpr (FP8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = min(seg_lo + tid + r * NWV * 64, seg_hi - 1);
      sk[r] = sbase[key_slot(slot_lo, key, a.cap)];
    }
  }
  uint4 buf[NF][4];
#pragma unroll
  for (int i = 0; i < NF; ++i) load(buf[i], i);
  if constexpr (FP8) {
    float smax = fmaxf(fmaxf(sk[0], sk[1]), fmaxf(sk[2], sk[3]));
    for (int key = seg_lo + tid + 4 * NWV * 64; key < seg_hi; key += NWV * 64)
      smax = fmaxf(smax, sbase[key_slot(slot_lo, key, a.cap)]);
    float qmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
    }
    smax = wave_max(smax);
    qmax = wave_max(qmax);
    if (lane == 0) {
      s_norm[0][wave] = smax;
      s_norm[1][wave] = qmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      smax = fmaxf(smax, s_norm[0][w]);
      qmax = fmaxf(qmax, s_norm[1][w]);
    }
    p_norm = pow2_norm(smax, 7);
    const float q_norm = pow2_norm(qmax, 15);
    logit_scale = a.scale / (q_norm * p_norm);  // exact: powers of two
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[j] = bf16x8_to_f16x8(qv[j], q_norm);
  }
  int t = 0;
  for (; t + NF - 1 < nt; t += NF) {
#pragma unroll
    for (int i = 0; i < NF; i += 2) step2(buf[i], buf[i + 1], t + i);
  }
#pragma unroll
  for (int i = 0; i < NF; i += 2)
    if (t + i < nt) step2(buf[i], buf[i + 1], t + i);

  app.store(a);
  // ---- this wave's slice of the result (m and l are identical in every wave of a group)
  l = rows_sum(l);
  if constexpr (MH == 2) {
    // the second group hands (m, l, acc) to the first through its own tile area; the
    // first group's first key is always valid, so its m is finite
    floatx4_t* comb = reinterpret_cast<floatx4_t*>(s_kv + (MNW + wsl) * 2 * WAVE_TILE);
    if (half == 1) {
      wave_lds_sync();  // this wave's last transposed reads stay before these writes
#pragma unroll
      for (int db = 0; db < 8; ++db) comb[db * 64 + lane] = acc[db];
      if (wsl == 0 && lane < MG) {
        s_ml[lane][0] = m;
        s_ml[lane][1] = l;
      }
    }
    __syncthreads();
    if (half == 1) return;
    const float m1 = s_ml[l16][0], l1 = s_ml[l16][1];
    const float mx = fmaxf(m, m1);
    const float f0 = exp2_fast(m - mx), f1 = exp2_fast(m1 - mx);  // m1 = -inf: f1 = 0
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = acc[db] * f0 + comb[db * 64 + lane] * f1;
    l = l * f0 + l1 * f1;
    m = mx;
  }
  if constexpr (FP8) {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] *= 1.0f / p_norm;  // exact: a power of two
  }
  if (k_u == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* o = a.out + (head0 + l16) * MD + DQ * wsl + 4 * lg;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4_t*>(o + 16 * db) = acc[db] * inv;
  } else {
    const size_t slot = (size_t)g_id;
    float* o = a.part_acc + (slot * MG + l16) * MD + DQ * wsl + 4 * lg;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4_t*>(o + 16 * db) = acc[db];
    if (wsl == 0 && lane < MG) {
      a.part_ml[(slot * MG + lane) * 2 + 0] = m;
      a.part_ml[(slot * MG + lane) * 2 + 1] = l;
    }
  }
}

// Finishes the units that were split over several work-groups; writes 0 for empty
// units.  One work-group per (unit, head): wave w takes partial slots w, w + 4, ...,
// with up to 16 slots' loads in flight per wave (so a unit of up to 64 partials costs
// one round of loads); lane l owns d = 8 l .. 8 l + 7.  Each wave keeps an online
// log-sum-exp, and the four wave states are combined through LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeBatch = 16;

__global__ void __launch_bounds__(kMergeThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
merge_units_kernel(DecodeArgs a) {
  __shared__ float s_ml[kMergeWaves][2];
  __shared__ __attribute__((aligned(16))) float s_o[kMergeWaves][MD];
  const int u = blockIdx.x / MG, h = blockIdx.x % MG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K0 = a.plan[u], K1 = a.plan[u + 1];
  const size_t head = ((size_t)(u / a.Hkv) * a.Hq + (size_t)(u % a.Hkv) * MG + h);
  float* out = a.out + head * MD;
  const int ks = K1 - K0;
  if (ks == 0) {  // no valid keys
    for (int d = tid; d < MD; d += kMergeThreads) out[d] = 0.0f;
    return;
  }
  if (ks == 1) return;  // written directly by the decode kernel
  const float* ml = a.part_ml + ((size_t)K0 * MG + h) * 2;
  const float4* acc =
      reinterpret_cast<const float4*>(a.part_acc + ((size_t)K0 * MG + h) * MD) + 2 * lane;
  const size_t ml_stride = (size_t)MG * 2, acc_stride4 = (size_t)MG * MD / 4;
  float M = -INFINITY, L = 0.0f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < ks; s0 += kMergeWaves * kMergeBatch) {
    float mb[kMergeBatch], lb[kMergeBatch];
    float4 va[kMergeBatch], vb[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int s = min(s0 + kMergeWaves * i, ks - 1);  // past the end: a valid slot, unused
      mb[i] = ml[s * ml_stride];
      lb[i] = ml[s * ml_stride + 1];
      va[i] = acc[s * acc_stride4];
      vb[i] = acc[s * acc_stride4 + 1];
    }
    float mnew = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + kMergeWaves * i < ks) mnew = fmaxf(mnew, mb[i]);
    const float f = M == -INFINITY ? 0.0f : exp2_fast(M - mnew);
    L *= f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= f;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      // no early exit: every load is consumed, so all of them are issued up front
      const float w = s0 + kMergeWaves * i < ks ? exp2_fast(mb[i] - mnew) : 0.0f;
      L = fmaf(lb[i], w, L);
      o[0] = fmaf(va[i].x, w, o[0]);
      o[1] = fmaf(va[i].y, w, o[1]);
      o[2] = fmaf(va[i].z, w, o[2]);
      o[3] = fmaf(va[i].w, w, o[3]);
      o[4] = fmaf(vb[i].x, w, o[4]);
      o[5] = fmaf(vb[i].y, w, o[5]);
      o[6] = fmaf(vb[i].z, w, o[6]);
      o[7] = fmaf(vb[i].w, w, o[7]);
    }
    M = mnew;
  }
  // a wave without slots (ks < 4) leaves M = -inf, L = 0, o = 0: weight 0 below
  if (lane == 0) {
    s_ml[wave][0] = M;
    s_ml[wave][1] = L;
  }
  float4* so = reinterpret_cast<float4*>(&s_o[wave][0]) + 2 * lane;
  so[0] = make_float4(o[0], o[1], o[2], o[3]);
  so[1] = make_float4(o[4], o[5], o[6], o[7]);
  __syncthreads();
  float Mall = s_ml[0][0];  // wave 0 always holds slot 0
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) Mall = fmaxf(Mall, s_ml[w][0]);
  float wt[kMergeWaves], Lall = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    wt[w] = exp2_fast(s_ml[w][0] - Mall);
    Lall = fmaf(s_ml[w][1], wt[w], Lall);
  }
  const float inv = 1.0f / Lall;
#pragma unroll
  for (int r = 0; r < MD / kMergeThreads; ++r) {
    const int d = tid + r * kMergeThreads;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) v = fmaf(s_o[w][d], wt[w], v);
    out[d] = v * inv;
  }
}

}  // namespace

bool decode_mfma_supported(int D, int G, bool k_eq_v) { return D == MD && G == MG && k_eq_v; }

size_t decode_mfma_workspace_bytes(int B, int Hkv) {
  const size_t units = (size_t)B * Hkv;
  const size_t slots = (size_t)kMfmaBlocks + units;  // >= sum of k_u, the grid size
  return slots * MG * MD * 4 + slots * MG * 2 * 4 + (units + 1) * 4;
}

hipError_t decode_mfma_launch(const DecodeArgs& a0, hipStream_t stream) {
  DecodeArgs a = a0;
  const long long R = (long long)a.B * a.Hkv;
  if (R <= 0) return hipSuccess;
  if (R > kMfmaMaxUnits) return hipErrorInvalidValue;
  a.n_blocks = kMfmaBlocks;
  // Work-groups with work: with R <= 3/4 NB at most R units are non-empty, the kernel
  // takes C = T / (NB - non-empty) and the sum of k_u stays <= NB; past that it takes
  // C = T / NB and the sum stays <= NB + R.  Work-groups u < R also carry unit u's append.
  const unsigned grid =
      (unsigned)(R <= kMfmaBlocks - kMfmaBlocks / 4 ? kMfmaBlocks : kMfmaBlocks + R);
  if (a.fp8)
    hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(grid), dim3(NWV * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<false>, dim3(grid), dim3(NWV * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_units_kernel, dim3((unsigned)(R * MG)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ga
