// decode_mfma.hip -- matrix-core split-KV decode for the K = V global geometry
// (head_dim 512, 16 query heads per KV head, one cached tensor used as keys and values).
//
// Why matrix cores here: 16 query heads share every key, so a key row of 1 KiB feeds
// 2 * 16 * 512 * 2 = 32 KFLOP (q.k and p.v): 32 flop/byte, above the fp32 vector ridge
// of MI355X (~157 TFLOP/s over 8 TB/s ~ 20 flop/byte), so a VALU kernel cannot reach
// the HBM roofline ("Gemma4-26B-A4B on Apple Silicon", Results, Break 4: 16 query heads
// on one shared K/V head, no separate value projection).
//
// Work partition: the chip gets NB work-groups' worth of keys (NB = the device's compute
// units, one work-group each), C = ceil(T / NB) keys each (T = valid keys of the whole
// batch, rounded to whole steps of the work-group's four waves), and every (batch row, KV
// head) unit u with n_u keys gets k_u = ceil(n_u / C) work-groups, each an equal share of
// that unit's keys.  The counts come from prefix sums computed on the device from
// ctx_lens / q_pos, so ragged contexts with few units (one KV head, batch 16-32) still
// spread evenly over every CU -- the failure mode of decode kernels that ignore key
// splitting ("Gemma 4 12B (unified multimodal)" record, item (4): 2 of 132 SMs busy) -- and
// no work-group ever switches units.  Sum k_u <= NB + units, the grid size.  A unit with
// k_u = 1 is written directly; the others leave one partial per work-group (slot =
// work-group index) for merge_units_kernel (log-sum-exp).  With a split size given, C is
// that size instead and the host sizes the grid for it.
//
// One work-group of 4 waves per CU, one wave per SIMD, and every wave works alone: wave w
// takes the work-group's steps w, w + 4, ... (bf16: one 16-key tile per step; fp8: two),
// with its own softmax state over the whole head_dim, so the key loop has no barrier and
// no exchange between waves.  Per step:
//   the step's rows sit in registers (16 load instructions, non-temporal: bf16 one 1 KiB
//     key row each, eight whole 128-byte lines; fp8 two rows of 512 codes each); they go to
//     the wave's LDS tiles row by row (fp8 codes widened exactly to bf16 on the way), each
//     row's registers refilling at once with the next step's row, so every wave keeps 16
//     loads in flight (a streaming probe on this chip: 6.5 TB/s with 16 per wave, 4.7 with
//     32);
//   S^T[16 keys][16 heads] = K[16][512] . Q^T[512][16] per tile with 16
//     v_mfma_f32_16x16x32_bf16: the A operand read back from the tile (lane: key l16,
//     d = 32 j + 8 lg + 0..7), Q^T read in the same d order from the unit's query rows in
//     LDS (lane: head l16);
//   the product leaves lane l with head l16 and keys 4 lg + 0..3, which is the B operand
//     layout of the P.V product, so the softmax runs in place (max and sum over the four
//     lane groups) and P goes to the matrix cores as bf16 hi + lo parts (~16 bits);
//   O^T[512][16] += V^T[512][keys] . P^T[keys][16 heads] with v_mfma_f32_16x16x32_bf16:
//     per 16-wide d block one (one tile: its keys in both halves of the k slots, against
//     P's hi and lo parts) or two (two tiles: one per P part), the A
//     operand from ds_read_b64_tr_b16 (lanes 4e..4e+3 of a 16-lane block read 16
//     consecutive d of key e, lane i then holds the 4 keys at column d0 + i); the K = V
//     row is read from HBM once and used for both products.
// LDS rows are 1 KiB with 16-byte chunk c of row r stored at chunk c ^ swz(r), which keeps
// the row writes, the A-operand reads and the transposed reads free of bank conflicts.
// At the end the four waves combine through LDS (each wave one quarter of head_dim) and the
// work-group writes its output or partial.  Softmax state per head is fp32 in log2 units:
// the reference is the wave's first maximum and stays fixed while no logit exceeds it by
// 64 (the accumulator then only ever sees the matrix cores); past that the wave continues
// with lazy rescaling (reference raised past +8).
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_mfma.h"
#include "ga_quant.h"
#include "ga_rope.h"

#include <type_traits>

namespace ga {
namespace {

constexpr int MD = 512;          // head_dim
constexpr int MG = 16;           // query heads per KV head
constexpr int TK = 16;           // keys per tile (the matrix-core operand height)
constexpr int NWV = kMfmaWaves;  // waves per work-group
constexpr int ROWB = MD * 2;     // LDS bytes per key row (bf16)
constexpr int TILEB = TK * ROWB;
constexpr int WAVE_LDS = 2 * TILEB;  // a wave's LDS: its tiles, and its accumulator at the end
constexpr float kRescaleLog2 = 8.0f;
// Fast-form headroom (log2 units): with the reference at the wave's first maximum, weights
// stay below 2^64, far inside fp32 (and bf16) range for the accumulator and the sum.
constexpr float kFastHeadroom = 64.0f;
static_assert(NWV * WAVE_LDS + MG * ROWB + 2 * (kMfmaMaxUnits + 1) * 4 + kMfmaMaxUnits * 4 +
                      NWV * MG * 2 * 4 + NWV * 32 * 4 + ROWB <=
                  160 * 1024,
              "LDS budget per work-group");
static_assert(WAVE_LDS >= 32 * 64 * 16, "a wave's LDS holds its accumulator at the end");

// LDS chunk swizzle (16-byte chunks, rows 0..15 of a tile): chunk c of row r sits at
// c ^ (2 r mod 16).  Measured on gfx950 (SQ_LDS_BANK_CONFLICT of each access pattern in
// isolation): no bank conflicts for the row writes, the A-operand reads (16 rows, one
// chunk each) and the transposed reads (4 rows x 32 bytes per 16 lanes).
__device__ __forceinline__ int swz(int r) { return (2 * r) & 15; }

// Keys per work-group, a multiple of the NWV steps a work-group starts on (wg_keys): then
// k_u = ceil(n_u / C) <= ceil(n_u / wg_keys), so the first wave of every work-group of a
// unit has a first step, and every work-group's result covers at least one key.
__device__ __forceinline__ int chunk_keys(int T, int NB, int wg_keys) {
  const int per = (T + NB - 1) / NB;
  return T > 0 ? (per + wg_keys - 1) / wg_keys * wg_keys : wg_keys;
}
// The smallest wg_keys of the kernels (bf16: one 16-key tile per step), which the host
// uses to bound the grid for a given split size.
constexpr int kMinWgKeys = NWV * TK;

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

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Rotary embedding of element d of a row at the angles of tab (the (cos, sin) pairs of one
// position): rotate-half pairs (i, i + MD/2) with i < nrot turn, the rest pass through.
// The same per-pair arithmetic as the RoPE + append kernel, so both give the same bits.
__device__ __forceinline__ uint16_t rope_at(const uint16_t* row, int d, int nrot,
                                            const double2* tab) {
  constexpr int H = MD / 2;
  const int i = d < H ? d : d - H;
  if (i >= nrot) return row[d];
  const double2 cs = tab[i];
  return d < H ? rope_first(row[i], row[i + H], cs.x, cs.y)
               : rope_second(row[i], row[i + H], cs.x, cs.y);
}

// FP8 with new_pos: the quantizing append fused in.  Wave 0 of every work-group quantizes
// its unit's new row (the same row quantizer as the quantizing append kernel, so the same
// codes and scale); the unit's first work-group stores them into the slot, and the wave
// whose step holds the appended key puts the widened codes and the scale into its tile and
// scale array in place of what it loaded from the slot.  A unit with no keys: work-group u
// appends its row directly.
// ROPE (bf16 caches): the rotary embedding at new_pos[b] fused in.  Every work-group
// rotates its unit's 16 query rows and new K row in LDS (from the same (cos, sin) table
// as the RoPE + append kernel); the unit's first work-group writes the rotated rows out
// (q_rot_out, and the K row into its cache slot), and the work-group holding the appended
// key puts the rotated row into its tile in place of the one it loaded from k_new.  A
// unit with no keys has no work-group of its own: work-group u writes its rows.
// CAP: the soft-cap is on (a separate instantiation: a condition inside the step is
// turned into selects, which evaluates the cap's exp and reciprocal when it is off).
template <bool FP8, bool ROPE, bool CAP>
__global__ void __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_mfma_kernel(DecodeArgs a) {
  static_assert(!(FP8 && ROPE), "RoPE is fused on bf16 caches only");
  // Tiles per step: bf16 one (16 load instructions of a whole 1 KiB row each); fp8 two
  // (8 instructions of two 512-code rows each per tile).  Either way a wave keeps NLS = 16
  // load instructions in flight.
  constexpr int TPS = FP8 ? 2 : 1;
  constexpr int STEP = TPS * TK;
  constexpr int NLS = 16;
  constexpr int WG_KEYS = NWV * STEP;
  // the unit's 16 query rows first, then the waves' tiles: the query rows then sit low
  // enough in LDS for every read of them to take its offset in the instruction
  __shared__ __attribute__((aligned(16))) char s_qkv[MG * ROWB + NWV * WAVE_LDS];
  char* const s_q = s_qkv;                // the unit's 16 query rows
  char* const s_kv = s_qkv + MG * ROWB;   // the waves' tiles
  __shared__ __attribute__((aligned(16))) float s_scl[NWV][32];  // fp8: the step's row scales
  __shared__ float s_ml[NWV][MG][2];
  __shared__ int s_n[kMfmaMaxUnits + 1];  // valid keys per unit, then their prefix sums
  __shared__ int s_k[kMfmaMaxUnits + 1];  // work-groups per unit, then their prefix sums
  __shared__ int s_slot[kMfmaMaxUnits];   // each unit's first slot
  __shared__ __attribute__((aligned(16))) uint16_t s_krot[ROPE ? MD : 8];  // rotated new K row
  __shared__ __attribute__((aligned(16))) uint8_t s_kq[FP8 ? MD : 16];      // its e4m3 codes
  __shared__ float s_kqs;                                                   // and scale

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uni(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.B * a.Hkv;
  // fused append: work-group u (< R <= grid) moves unit u's new row, stored at its end;
  // the row's position is requested here, ahead of everything, and used only there
  const int app_u = blockIdx.x < R ? blockIdx.x : 0;
  const int app_pos = a.new_pos && blockIdx.x < R ? a.new_pos[app_u / a.Hkv] : -1;

  // ---- the partition (every work-group computes it; work-group 0 also publishes it):
  // each unit's key range (its first slot kept for the unit's own work-groups), then wave 0
  // alone forms both prefix sums (two barriers).
  {
    // every thread's loads first (a unit past R re-reads row 0), then their ranges
    constexpr int UPT = (kMfmaMaxUnits + NWV * 64 - 1) / (NWV * 64);
    int cx[UPT], qx[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NWV * 64;
      const int b = u < R ? u / a.Hkv : 0;
      cx[i] = a.ctx[b];
      qx[i] = a.q_pos[b];
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NWV * 64;
      if (u < R) {
        const RowRange rr = row_range(cx[i], qx[i], a.window, a.kind, a.cap, a.max_keys);
        s_n[u + 1] = rr.n;
        s_slot[u] = rr.slot_lo;
      }
    }
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
    int C;
    if (a.split_keys > 0) {
      // a given split size (rounded up to whole work-group starts): the host sized the
      // grid for it
      C = (a.split_keys + WG_KEYS - 1) / WG_KEYS * WG_KEYS;
    } else {
      // k_u = ceil(n_u / C) <= n_u / C + 1, so with C = T / (NB - R') (R' non-empty units)
      // the work-groups with work never exceed NB: all of them are resident at once.
      const int nb_eff =
          a.n_blocks - nonempty >= a.n_blocks / 4 ? a.n_blocks - nonempty : a.n_blocks;
      C = chunk_keys(total, nb_eff, WG_KEYS);
    }
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
  AppendRow app;  // (its slot is given at the store, from app_pos)
  app.load_unplaced(a, app_u / a.Hkv, app_u % a.Hkv, tid, !ROPE && !FP8 && blockIdx.x < R);
  auto app_store = [&]() {
    app.place(a, appended_slot_at(a, app_pos), tid);
    app.store(a);
  };
  // FP8: the quantizing append of unit uu's new row w (lane: values 8 lane .. 8 lane + 7)
  // by wave 0 (codes in LDS and, when store, in the cache); every lane of wave 0 calls it
  auto new_row = [&](int uu) { return reinterpret_cast<const uint4*>(a.k_new + (size_t)uu * MD)[lane]; };
  auto quant_append = [&](int uu, const uint4& w, bool store, int slot) {
    float sc;
    const uint2 c8 = quantize_row_e4m3(w, true, &sc);
    reinterpret_cast<uint2*>(s_kq)[lane] = c8;
    if (lane == 0) s_kqs = sc;
    if (store && slot >= 0) {
      reinterpret_cast<uint2*>(a.k8_dst + ((size_t)uu * a.cap + slot) * MD)[lane] = c8;
      if (lane == 0) a.ks_dst[(size_t)uu * a.cap + slot] = sc;
    }
  };
  // ROPE: rows of a unit without work-groups (no valid keys), by work-group u, directly
  // from global memory
  auto rope_unit_direct = [&](int uu) {
    const int bb = uu / a.Hkv, gg = uu % a.Hkv, half = a.rope_dim / 2;
    const double2* tab = reinterpret_cast<const double2*>(a.rope_table) + (size_t)bb * half;
    const size_t h0 = (size_t)bb * a.Hq + (size_t)gg * MG;
    for (int e = tid; e < MG * MD; e += NWV * 64)
      a.q_rot_out[(h0 + e / MD) * MD + e % MD] = rope_at(a.q + (h0 + e / MD) * MD, e % MD, half, tab);
    const int slot = appended_slot(a, bb);
    if (slot >= 0)
      for (int d = tid; d < MD; d += NWV * 64)
        a.k_dst[((size_t)uu * a.cap + slot) * MD + d] = rope_at(a.k_new + (size_t)uu * MD, d, half, tab);
  };
  const int g_id = blockIdx.x;
  if constexpr (ROPE) {
    if (g_id < R && s_k[g_id + 1] == s_k[g_id]) rope_unit_direct(g_id);
  }
  if constexpr (FP8) {
    if (a.new_pos && g_id < R && s_k[g_id + 1] == s_k[g_id] && wave == 0)
      quant_append(g_id, new_row(g_id), true, appended_slot(a, g_id / a.Hkv));
  }
  if (g_id >= s_k[R]) {
    app_store();
    return;
  }
  // unit of this work-group: the u with s_k[u] <= g_id < s_k[u + 1]
  int u;
  {
    int lo_u = 0, hi_u = R - 1;
    while (lo_u < hi_u) {
      const int mid = (lo_u + hi_u) >> 1;
      if (s_k[mid + 1] > g_id) hi_u = mid; else lo_u = mid + 1;
    }
    u = uni(lo_u);
  }
  const int n_u = uni(s_n[u + 1] - s_n[u]);
  const int k_u = uni(s_k[u + 1] - s_k[u]);
  const int part = g_id - uni(s_k[u]);
  const int per = ((n_u + k_u - 1) / k_u + WG_KEYS - 1) / WG_KEYS * WG_KEYS;
  const int seg_lo = part * per;
  const int seg_hi = min(n_u, seg_lo + per);  // non-empty: (k_u - 1) * per < n_u
  const int nsteps = (seg_hi - seg_lo + STEP - 1) / STEP;
  // wave w takes the segment's steps w, w + NWV, ...; every wave has one (per >= WG_KEYS)
  // except in a unit's last work-group
  const int my_steps = wave < nsteps ? (nsteps - wave + NWV - 1) / NWV : 0;

  const int b = u / a.Hkv, g = u % a.Hkv;
  const int slot_lo = uni(s_slot[u]);
  // the appended token's position, requested ahead of the query rows and waited for with
  // them (a zero the compiler cannot see through keeps it a vector load, not one waited
  // for at once)
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  const int new_pos_b = a.new_pos ? a.new_pos[b + zero] : -1;
  const size_t head0 = (size_t)b * a.Hq + (size_t)g * MG;
  const int cap = a.cap;
  // ROPE: the unit's new K row, unrotated, to LDS, and the (cos, sin) pairs this thread
  // turns (pair i = tid % half of rows tid / half, tid / half + groups, ...)
  const int rhalf = ROPE ? a.rope_dim / 2 : 0;
  const int rgroups = rhalf > 0 ? (NWV * 64) / rhalf : 0;
  double2 rcs = make_double2(1.0, 0.0);
  if constexpr (ROPE) {
    if (tid < MD / 8)
      *reinterpret_cast<uint4*>(s_krot + 8 * tid) =
          reinterpret_cast<const uint4*>(a.k_new + (size_t)u * MD)[tid];
    if (tid < rgroups * rhalf)
      rcs = reinterpret_cast<const double2*>(a.rope_table)[(size_t)b * rhalf + tid % rhalf];
  }

  // FP8: the unit's new row requested ahead of the query rows (quantized once they are in)
  uint4 kw = make_uint4(0, 0, 0, 0);
  if constexpr (FP8) {
    if (a.new_pos && wave == 0) kw = new_row(u);
  }
  // the unit's 16 query rows to LDS in the key rows' layout (row = head, chunk c at
  // c ^ swz(row)): the Q^T operand is read from there like the K operand (lane: head l16,
  // d = 32 j + 8 lg + 0..7), which leaves the registers to the rows in flight
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + head0 * MD);
#pragma unroll
    for (int k = 0; k < MG * MD / 8 / (NWV * 64); ++k) {
      const int idx = tid + k * NWV * 64, r = idx >> 6, c = idx & 63;
      *reinterpret_cast<uint4*>(s_q + r * ROWB + ((c ^ swz(r)) * 16)) = qp[idx];
    }
  }
  const int new_slot = uni(appended_slot_at(a, new_pos_b));  // fused append: from k_new
  if constexpr (FP8) {
    // the unit's new row quantized (stored by the unit's first work-group); measured
    // 1 us faster per launch here than after the first rows are requested
    if (a.new_pos && wave == 0) quant_append(u, kw, part == 0, new_slot);
  }

  // ---- loads.  Tile h of step t (of this wave: the segment's step wave + NWV t) holds the
  // segment's keys seg_lo + STEP (wave + NWV t) + 16 h + 0..15.  Keys past the segment's end
  // re-read its last key (a valid row, masked), so every load is unconditional.
  // ROPE / FP8: the appended key's index in the unit's range (-1 when it has none)
  int new_key = -1;
  if ((ROPE || FP8) && new_slot >= 0) {
    const int nk = new_slot - slot_lo < 0 ? new_slot - slot_lo + cap : new_slot - slot_lo;
    if (nk < n_u) new_key = nk;
  }
  const char* kmem = FP8 ? reinterpret_cast<const char*>(a.k8) : reinterpret_cast<const char*>(a.k);
  constexpr int CROWB = FP8 ? MD : MD * 2;  // bytes per cached row
  const char* kunit = kmem + (size_t)u * cap * CROWB;
  const char* knew = a.new_pos ? reinterpret_cast<const char*>(a.k_new) + (size_t)u * ROWB
                               : kunit;
  const float* sunit = FP8 ? a.k_scale + (size_t)u * cap : nullptr;
  auto slot_of = [&](int key) { return key_slot(slot_lo, key < seg_hi ? key : seg_hi - 1, cap); };
  auto key0 = [&](int t) { return seg_lo + STEP * (wave + NWV * t); };
  // one step's registers: NLS load instructions (bf16: 16 rows of one tile; fp8: 8 row
  // pairs of each of two tiles) and (fp8) the row scale of key lane % 32 of the step
  struct Regs {
    uint4 r[NLS];
    float sc;
  };
  // fp8: a step whose keys are all inside the segment and on consecutive slots (no ring
  // wrap) -- every step but a few -- has its row pairs at kunit + (first + 2 j) * CROWB,
  // i.e. base + 1024 j + 16 lane: one base per step instead of two slots per load
  // (1.7 us faster per launch on the 12B fp8 global layer; the same on bf16 rows measured
  // 10 us slower, the compiler then keeping the accumulator partly outside the AGPRs).
  auto step_first = [&](int k0) { return uni(slot_of(k0)); };
  auto step_contig = [&](int k0, int first) {
    return FP8 && k0 + STEP <= seg_hi && first + STEP <= cap;
  };
  auto load_row_at = [&](Regs& t, int j, const char* base) __attribute__((always_inline)) {
    t.r[j] = stream_load(reinterpret_cast<const uint4*>(base + 1024 * j) + lane);
  };
  auto load_scale_at = [&](Regs& t, int first) __attribute__((always_inline)) {
    if constexpr (FP8) t.sc = sunit[first + (lane & 31)];
  };
  auto load_row = [&](Regs& t, int j, int k0) __attribute__((always_inline)) {
    if constexpr (FP8) {
      // rows 2 j and 2 j + 1 of the step: lanes 0..31 the first, 32..63 the second
      const int sa = uni(slot_of(k0 + 2 * j)), sb = uni(slot_of(k0 + 2 * j + 1));
      const char* row = kunit + (size_t)(lane < 32 ? sa : sb) * CROWB;
      t.r[j] = stream_load(reinterpret_cast<const uint4*>(row) + (lane & 31));
    } else {
      const int slot = uni(slot_of(k0 + j));
      const char* row = slot == new_slot ? knew : kunit + (size_t)slot * CROWB;
      t.r[j] = stream_load(reinterpret_cast<const uint4*>(row) + lane);
    }
  };
  auto load_scale = [&](Regs& t, int k0) __attribute__((always_inline)) {
    if constexpr (FP8) t.sc = sunit[slot_of(k0 + (lane & 31))];
  };
  char* my_tiles = s_kv + wave * WAVE_LDS;
  // load instruction j of a step to LDS (row r of tile r / 16, 16-byte chunk c at c ^ swz)
  auto put_row = [&](const Regs& t, int j) __attribute__((always_inline)) {
    if constexpr (FP8) {
      // lane widens 16 codes (d = 16 m + 0..15, m = lane % 32) of step row 2 j + lane / 32
      // to the two chunks 2 m and 2 m + 1, storing first the one that keeps 8 / 16
      // consecutive lanes on distinct banks
      // (the swap picks the source words before widening: four selects per row pair)
      const int m = lane & 31, fb = ((m >> 2) ^ (m >> 3)) & 1;
      const int rs = 2 * j + (lane >> 5), r = rs & 15, sw = swz(r);
      const uint4 v = t.r[j];
      const uint4 first = e4m3x8_to_bf16x8(fb ? v.z : v.x, fb ? v.w : v.y);
      const uint4 second = e4m3x8_to_bf16x8(fb ? v.x : v.z, fb ? v.y : v.w);
      char* row = my_tiles + (rs >> 4) * TILEB + r * ROWB;
      *reinterpret_cast<uint4*>(row + ((2 * m + fb) ^ sw) * 16) = first;
      *reinterpret_cast<uint4*>(row + ((2 * m + 1 - fb) ^ sw) * 16) = second;
    } else {
      *reinterpret_cast<uint4*>(my_tiles + j * ROWB + ((lane ^ swz(j)) * 16)) = t.r[j];
    }
  };
  auto put_scale = [&](const Regs& t) __attribute__((always_inline)) {
    if constexpr (FP8) {
      if (lane < 32) s_scl[wave][lane] = t.sc;
    }
  };
  // The step's registers to LDS, each load instruction's register refilled with the same
  // instruction of step t_next as soon as its row is stored: the wave keeps NLS loads in
  // flight at all times (more per wave measured slower on this chip).  The scheduling
  // barriers keep every store before the next row's refill; without them the compiler
  // stores all of a step's rows first, which waits for every load in flight.
  auto cycle = [&](Regs& t, int t_next) __attribute__((always_inline)) {
    const int k0 = key0(t_next);
    put_scale(t);
    if constexpr (FP8) {
      const int first = step_first(k0);
      if (step_contig(k0, first)) {
        const char* base = kunit + (size_t)first * CROWB;
        load_scale_at(t, first);
#pragma unroll
        for (int j = 0; j < NLS; ++j) {
          put_row(t, j);
          load_row_at(t, j, base);
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
    }
    load_scale(t, k0);
#pragma unroll
    for (int j = 0; j < NLS; ++j) {
      put_row(t, j);
      load_row(t, j, k0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto put = [&](const Regs& t) __attribute__((always_inline)) {
    put_scale(t);
#pragma unroll
    for (int j = 0; j < NLS; ++j) put_row(t, j);
  };
  // per-lane LDS offsets: A operand (row l16, chunk 4 jj + lg for jj = j % 4; j / 4 adds
  // 16 chunks) and transposed reads (row 4 lg + l16 / 4, chunk 2 e + (l16 / 2) % 2 of the
  // d block db = 8 (db / 8) + e, byte 8 (l16 % 2) in it)
  int a_off[4], t_off[8];
  {
    const int sa = swz(l16);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) a_off[jj] = l16 * ROWB + ((4 * jj + lg) ^ sa) * 16;
    const int rr = 4 * lg + (l16 >> 2), st = swz(rr), hh = (l16 >> 1) & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) t_off[e] = rr * ROWB + ((2 * e + hh) ^ st) * 16 + (l16 & 1) * 8;
  }

  floatx4_t acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;

  // One step from the LDS tiles.  The reference m per head is the wave's first maximum;
  // in the fast form (SAFE = false) it never moves afterwards, so the accumulator is only
  // ever touched by the matrix cores, and a step whose maximum exceeds m + kFastHeadroom
  // (where 2^(x - m) could leave the fp32 range) returns false before using any of its
  // values; the caller then finishes in the safe form, which rescales the accumulator
  // whenever the maximum grows by more than kRescaleLog2 (lazy rescaling).
  auto compute = [&](auto safe_tag, int t) __attribute__((always_inline)) -> bool {
    constexpr bool SAFE = decltype(safe_tag)::value;
    const int k0 = key0(t);
    // S^T per tile: 16 products over head_dim, in two chains per tile (even / odd j); the
    // K and Q operands are read a group of QG products ahead
    floatx4_t sc2[TPS][2];
#pragma unroll
    for (int h = 0; h < TPS; ++h) sc2[h][0] = sc2[h][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int QG = 2;
    uint4 kk[2][TPS][QG], qq[2][QG];
    auto read_k = [&](int grp, uint4(&x)[TPS][QG], uint4(&z)[QG]) {
#pragma unroll
      for (int jj = 0; jj < QG; ++jj) {
        const int j = grp * QG + jj;
        const int off = a_off[j & 3] + 256 * (j >> 2);
#pragma unroll
        for (int h = 0; h < TPS; ++h)
          x[h][jj] = *reinterpret_cast<const uint4*>(my_tiles + h * TILEB + off);
        z[jj] = *reinterpret_cast<const uint4*>(s_q + off);
      }
    };
    read_k(0, kk[0], qq[0]);
#pragma unroll
    for (int grp = 0; grp < 16 / QG; ++grp) {
      const int nx = (grp + 1) & 1;
      if (grp + 1 < 16 / QG) read_k(grp + 1, kk[nx], qq[nx]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < QG; ++jj)
#pragma unroll
        for (int h = 0; h < TPS; ++h)
          sc2[h][jj & 1] = mfma_k32(kk[grp & 1][h][jj], qq[grp & 1][jj], sc2[h][jj & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // softmax: lane holds head l16, keys k0 + 16 h + 4 lg + e of tile h
    float ks[TPS][4];
    if constexpr (FP8) {  // the keys' row scales
#pragma unroll
      for (int h = 0; h < TPS; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(&s_scl[wave][16 * h + 4 * lg]);
        ks[h][0] = v.x; ks[h][1] = v.y; ks[h][2] = v.z; ks[h][3] = v.w;
      }
    }
    float x[TPS][4], mx = -INFINITY;
    // without the cap the logit in log2 units is s * (scale log2 e) (* the row scale)
    const float s2 = CAP ? a.scale : a.scale * kLog2e;
#pragma unroll
    for (int h = 0; h < TPS; ++h) {
      const floatx4_t sv = sc2[h][0] + sc2[h][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = sv[e] * s2;
        if constexpr (FP8) v *= ks[h][e];
        if constexpr (CAP) v = softcap_tanh(v, a.softcap, a.inv_softcap) * kLog2e;
        x[h][e] = v;
      }
    }
    if (k0 + STEP > seg_hi) {  // the segment's last step: keys past its end weigh 0
      asm volatile("");  // (a branch, not selects evaluated on every step)
#pragma unroll
      for (int h = 0; h < TPS; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k0 + TK * h + 4 * lg + e >= seg_hi) x[h][e] = -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < TPS; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, x[h][e]);
    mx = rows_max(mx);  // over the step's keys (four lane groups)
    if constexpr (SAFE) {
      if (mx > m + kRescaleLog2) {
        const float f = exp2_fast(m - mx);  // 0 while m = -inf
        l *= f;
#pragma unroll
        for (int d = 0; d < 32; ++d) acc[d] *= f;
        m = mx;
      }
    } else {
      if (__ballot(m != -INFINITY && mx > m + kFastHeadroom) != 0) return false;
      if (m == -INFINITY) m = mx;  // the wave's first step (the accumulator is still 0)
    }
    // every step holds at least one valid key, so m is finite from the first step on
    const float mref = m == -INFINITY ? 0.0f : m;
    float p[TPS][4];
#pragma unroll
    for (int h = 0; h < TPS; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[h][e] = exp2_fast(x[h][e] - mref);
        l += p[h][e];
        if constexpr (FP8) p[h][e] *= ks[h][e];  // K = V: the value row's scale is the key's
      }
    // P^T operands (lane: head l16, keys 4 lg + 0..3 of each tile), bf16 hi + lo parts
    uint32_t ph[2 * TPS], pl[2 * TPS];
#pragma unroll
    for (int h = 0; h < TPS; ++h)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t hv = pack_bf16x2(p[h][2 * k], p[h][2 * k + 1]);
        ph[2 * h + k] = hv;
        pl[2 * h + k] = pack_bf16x2(p[h][2 * k] - bf16_lo(hv), p[h][2 * k + 1] - bf16_hi(hv));
      }
    // O^T += V^T P^T per 16-wide d block with v_mfma_f32_16x16x32_bf16: one tile -> the
    // tile's transposed read in both halves of the k slots (8 lg + 0..3 and 8 lg + 4..7:
    // keys 4 lg + 0..3), against P's hi part in the first half and its lo part in the
    // second, so one product covers both parts (on gfx950 the 16x16x16 form costs as many
    // cycles as this one); two tiles -> both tiles (k slots 8 lg + 0..3 = tile 0's keys
    // 4 lg + 0..3, 8 lg + 4..7 = tile 1's), once for P's hi and once for its lo part.
    // The V^T operands are read a group of VG blocks ahead.
    constexpr int VG = 4;
    uint4 vv[2][VG];
    auto read_v = [&](int grp, uint4(&y)[VG]) {
#pragma unroll
      for (int k = 0; k < VG; ++k) {
        const int db = grp * VG + k;
        const int off = t_off[db & 7] + 256 * (db >> 3);
        const short4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(my_tiles + off));
        short4_t vb = va;
        if constexpr (TPS == 2)
          vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(my_tiles + TILEB + off));
        y[k] = cat4(va, vb);
      }
    };
    read_v(0, vv[0]);
#pragma unroll
    for (int grp = 0; grp < 32 / VG; ++grp) {
      if (grp + 1 < 32 / VG) read_v(grp + 1, vv[(grp + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int part2 = 0; part2 < TPS; ++part2)
#pragma unroll
        for (int k = 0; k < VG; ++k) {
          const int db = grp * VG + k;
          if constexpr (TPS == 2) {
            const uint32_t* pp = part2 == 0 ? ph : pl;
            acc[db] = mfma_k32(vv[grp & 1][k], make_uint4(pp[0], pp[1], pp[2], pp[3]), acc[db]);
          } else {
            acc[db] = mfma_k32(vv[grp & 1][k], make_uint4(ph[0], ph[1], pl[0], pl[1]), acc[db]);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    return true;
  };

  // ---- the key loop: the current step's rows sit in registers; per step they go to LDS
  // row by row, each row's registers refilling with the next step's row, and the step is
  // computed from LDS.  The wave's last step only goes to LDS.
  Regs buf;
  load_scale(buf, key0(0));
#pragma unroll
  for (int j = 0; j < NLS; ++j) load_row(buf, j, key0(0));  // (a wave without steps: unused)
  __syncthreads();  // the query rows (and the quantized new row) are in LDS
  if constexpr (ROPE) {
    // rotate in place: rows 0..15 the query rows (swizzled chunks), row 16 the K row
    if (tid < rgroups * rhalf) {
      const int i = tid % rhalf;
      for (int r = tid / rhalf; r <= MG; r += rgroups) {
        uint16_t* e0;
        uint16_t* e1;
        if (r < MG) {
          char* row = s_q + r * ROWB;
          e0 = reinterpret_cast<uint16_t*>(row + ((i / 8) ^ swz(r)) * 16) + i % 8;
          e1 = reinterpret_cast<uint16_t*>(row + (((i + MD / 2) / 8) ^ swz(r)) * 16) + (i + MD / 2) % 8;
        } else {
          e0 = s_krot + i;
          e1 = s_krot + i + MD / 2;
        }
        const uint16_t x0 = *e0, x1 = *e1;
        *e0 = rope_first(x0, x1, rcs.x, rcs.y);
        *e1 = rope_second(x0, x1, rcs.x, rcs.y);
      }
    }
    __syncthreads();
    if (part == 0) {
      // the unit's first work-group: rotated q out, rotated K row into its slot (no
      // reader in this launch takes that slot from the cache)
      for (int idx = tid; idx < MG * MD / 8; idx += NWV * 64) {
        const int r = idx / (MD / 8), c = idx % (MD / 8);
        reinterpret_cast<uint4*>(a.q_rot_out + (head0 + r) * MD)[c] =
            *reinterpret_cast<const uint4*>(s_q + r * ROWB + (c ^ swz(r)) * 16);
      }
      if (new_slot >= 0 && tid < MD / 8)
        reinterpret_cast<uint4*>(a.k_dst + ((size_t)u * cap + new_slot) * MD)[tid] =
            *reinterpret_cast<const uint4*>(s_krot + 8 * tid);
    }
  }
  // one step: 0 to go on, 1 when it was the wave's last, 2 when the fast form stopped on it
  // (its tiles are in LDS)
  auto body = [&](auto safe_tag, int t) __attribute__((always_inline)) -> int {
    wave_lds_sync();  // the previous step's LDS reads stay before these writes
    const bool last = t + 1 >= my_steps;
    if (last) put(buf); else cycle(buf, t + 1);
    if constexpr (ROPE) {
      // the appended key's row came from k_new unrotated: the rotated one replaces it
      const int j = new_key - key0(t);
      if (new_key >= 0 && j >= 0 && j < TK && new_key < seg_hi)
        *reinterpret_cast<uint4*>(my_tiles + j * ROWB + ((lane ^ swz(j)) * 16)) =
            *reinterpret_cast<const uint4*>(s_krot + 8 * lane);
    }
    if constexpr (FP8) {
      // the appended key's slot may still hold the row it replaces (any bits, NaN codes
      // included): its codes (widened) and scale from the quantized new row instead, also
      // in the rows past the segment's end, which re-read the segment's last key (masked,
      // but a NaN would survive the zero weight)
      const int j = new_key - key0(t);
      if (new_key >= 0 && j >= 0 && j < STEP && new_key < seg_hi) {
        const uint2 c8 = reinterpret_cast<const uint2*>(s_kq)[lane];
        const uint4 wide = e4m3x8_to_bf16x8(c8.x, c8.y);
        const int j_end = new_key == seg_hi - 1 ? STEP : j + 1;
        for (int jj = j; jj < j_end; ++jj) {
          const int r = jj & 15;
          *reinterpret_cast<uint4*>(my_tiles + (jj >> 4) * TILEB + r * ROWB +
                                    ((lane ^ swz(r)) * 16)) = wide;
          if (lane == 0) s_scl[wave][jj] = s_kqs;
        }
      }
    }
    wave_lds_sync();
    if (!compute(safe_tag, t)) return 2;
    return last ? 1 : 0;
  };
  const std::integral_constant<bool, false> fast;
  const std::integral_constant<bool, true> safe;
  int t = 0, st = 1;
  for (; t < my_steps; ++t)
    if ((st = body(fast, t)) != 0) break;
  if (st == 2) {
    // finish in the safe form: the step that stopped (its tiles are in LDS), then the rest
    compute(safe, t);
    for (++t; t < my_steps; ++t)
      if (body(safe, t) != 0) break;
  }

  app_store();
  // ---- combine the waves: each leaves (m, l) per head and its accumulator (in its own
  // tile area), then wave w combines d blocks 8 w .. 8 w + 7 of all four
  l = rows_sum(l);
  wave_lds_sync();
  floatx4_t* mine = reinterpret_cast<floatx4_t*>(s_kv + wave * WAVE_LDS);
#pragma unroll
  for (int db = 0; db < 32; ++db) mine[db * 64 + lane] = acc[db];
  if (lg == 0) {
    s_ml[wave][l16][0] = m;
    s_ml[wave][l16][1] = l;
  }
  __syncthreads();
  float fw[NWV], M = -INFINITY, L = 0.0f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) M = fmaxf(M, s_ml[w][l16][0]);
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const float mw = s_ml[w][l16][0];
    fw[w] = mw == -INFINITY ? 0.0f : exp2_fast(mw - M);  // a wave without keys: weight 0
    L = fmaf(s_ml[w][l16][1], fw[w], L);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int dd = 0; dd < 32 / NWV; ++dd) {
    const int db = (32 / NWV) * wave + dd;
    floatx4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w)
      o += reinterpret_cast<const floatx4_t*>(s_kv + w * WAVE_LDS)[db * 64 + lane] * fw[w];
    const int d = 16 * db + 4 * lg;
    if (k_u == 1) {
      *reinterpret_cast<floatx4_t*>(a.out + (head0 + l16) * MD + d) = o * inv;
    } else {
      // non-temporal: read once, by the merge, most often on another XCD (the step's
      // 48 layers 2.117-2.118 -> 2.113-2.115 ms, three alternating pairs)
      __builtin_nontemporal_store(
          o, reinterpret_cast<floatx4_t*>(a.part_acc + ((size_t)g_id * MG + l16) * MD + d));
    }
  }
  if (k_u > 1 && wave == 0 && lg == 0) {
    a.part_ml[((size_t)g_id * MG + l16) * 2 + 0] = M;
    a.part_ml[((size_t)g_id * MG + l16) * 2 + 1] = L;
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
      const float w =
          s0 + kMergeWaves * i < ks && mb[i] != -INFINITY ? exp2_fast(mb[i] - mnew) : 0.0f;
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
    wt[w] = s_ml[w][0] == -INFINITY ? 0.0f : exp2_fast(s_ml[w][0] - Mall);
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

size_t decode_mfma_workspace_bytes(long long grid, int units) {
  const size_t slots = (size_t)grid;  // one partial per work-group
  // partials and the plan [units + 1]
  return slots * MG * MD * 4 + slots * MG * 2 * 4 + ((size_t)units + 1) * 4;
}

long long decode_mfma_grid(int units, int n_blocks, int split_keys, int max_keys) {
  if (split_keys > 0) {
    // every unit at most ceil(max_keys / C) work-groups, C the split size rounded up to
    // whole work-group starts (as the kernel rounds it)
    const long long c = ((long long)split_keys + kMinWgKeys - 1) / kMinWgKeys * kMinWgKeys;
    const long long per_unit = ((long long)max_keys + c - 1) / c;
    return (long long)units * (per_unit > 0 ? per_unit : 1);
  }
  // Work-groups with work: with R <= 3/4 NB at most R units are non-empty, the kernel
  // takes C = T / (NB - non-empty) and the sum of k_u stays <= NB; past that it takes
  // C = T / NB and the sum stays <= NB + R.  Work-groups u < R also carry unit u's append.
  return units <= n_blocks - n_blocks / 4 ? n_blocks : (long long)n_blocks + units;
}

hipError_t decode_mfma_launch(const DecodeArgs& a0, hipStream_t stream) {
  if (a0.B <= 0) return hipSuccess;
  // batches of more than kMfmaMaxUnits units run as several launches of whole rows (the
  // plan lives in LDS); the workspace is reused in stream order
  const int rows = a0.launch_rows > 0 ? a0.launch_rows : kMfmaMaxUnits / a0.Hkv;
  if (rows < 1 || (long long)rows * a0.Hkv > kMfmaMaxUnits) return hipErrorInvalidValue;
  for (int b0 = 0; b0 < a0.B; b0 += rows) {
    DecodeArgs a = a0;
    a.B = min(rows, a0.B - b0);
    const size_t qo = (size_t)b0 * a0.Hq * MD, unit0 = (size_t)b0 * a0.Hkv;
    a.q += qo;
    a.out += qo;
    a.ctx += b0;
    a.q_pos += b0;
    if (a.fp8) {
      a.k8 += unit0 * a0.cap * MD;
      a.v8 = a.k8;
      a.k_scale += unit0 * a0.cap;
      a.v_scale = a.k_scale;
    } else {
      a.k += unit0 * a0.cap * MD;
      a.v = a.k;
    }
    if (a.new_pos) {
      a.new_pos += b0;
      a.k_new += unit0 * MD;
      if (a.k_dst) a.k_dst += unit0 * a0.cap * MD;
      if (a.k8_dst) {
        a.k8_dst += unit0 * a0.cap * MD;
        a.ks_dst += unit0 * a0.cap;
      }
    }
    if (a.rope) {
      a.q_rot_out += qo;
      if (a.rope_table) a.rope_table += (size_t)b0 * a0.rope_dim;  // rope_dim / 2 pairs a row
    }
    const long long R = (long long)a.B * a.Hkv;
    const long long grid = decode_mfma_grid((int)R, a.n_blocks, a.split_keys, a.max_keys);
    if (grid < R || grid > (1LL << 31) - 1) return hipErrorInvalidValue;
    if (a.fp8 && a.rope) return hipErrorInvalidValue;  // (the plan never asks for it)
    const dim3 g3((unsigned)grid), b3(NWV * 64);
    const bool cap = a.softcap > 0.0f;
    if (a.fp8) {
      if (cap) hipLaunchKernelGGL((decode_mfma_kernel<true, false, true>), g3, b3, 0, stream, a);
      else hipLaunchKernelGGL((decode_mfma_kernel<true, false, false>), g3, b3, 0, stream, a);
    } else if (a.rope) {
      if (cap) hipLaunchKernelGGL((decode_mfma_kernel<false, true, true>), g3, b3, 0, stream, a);
      else hipLaunchKernelGGL((decode_mfma_kernel<false, true, false>), g3, b3, 0, stream, a);
    } else {
      if (cap) hipLaunchKernelGGL((decode_mfma_kernel<false, false, true>), g3, b3, 0, stream, a);
      else hipLaunchKernelGGL((decode_mfma_kernel<false, false, false>), g3, b3, 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_units_kernel, dim3((unsigned)(R * MG)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ga
