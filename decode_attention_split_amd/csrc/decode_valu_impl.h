// decode_valu_impl.h -- split-KV flash-decode on the vector ALUs (gfx950, wave64).
//
// Kernel templates and launchers; decode_valu_d{128,256,512}.hip each instantiate
// valu_launch_d for one head dim (compiled in parallel), decode_valu.hip dispatches.
//
// One work-group handles one split (a run of split_keys consecutive valid keys) of one
// (batch row, KV head).  Inside a wave, aligned groups of L lanes each own one key per
// step: lane j of a group holds the elements d = 8 * (c * L + j) + e (c < D / (8 L),
// e < 8) of that key's row, loaded straight from HBM with 16-byte loads (a group reads
// 16 L contiguous bytes per load, a full row over D / (8 L) loads).  The G query heads
// that share the KV head stay in registers as packed bf16, so q . k is v_dot2 on the raw
// bf16 data with fp32 accumulation, finished by a DPP butterfly over the group.  Every
// group keeps its own online-softmax state (m, l, acc[G][D / L]) and the groups and
// waves are merged once at the end, so the key loop has no barrier and no LDS traffic:
// each lane consumes exactly the bytes it loaded, and staging through LDS would only add
// a write and a read per byte.  With K = V the row loaded for the logits is the row
// used for the values (read once, used twice).
//
// Softmax runs in log2 units: s2 = log2(e) * cap(scale * q.k).  The running max is only
// raised when a logit exceeds it by more than kRescaleLog2 (2^8), so the accumulator
// rescale (G * D / L multiplies) happens a handful of times per group rather than per
// key; exp2(s2 - m) <= 2^8 keeps everything well inside fp32.  The result is unchanged:
// (m, l, acc) stay mutually consistent whatever reference m is used.
//
// Definition followed: "Gemma support" pull request, Summary (soft-capping, sliding
// window, head sizes 256/512, K = V) and Performance (split decode attention); the key
// range is ga::row_range ("Gemma 4 12B (unified multimodal)" record: exactly w entries).
#pragma once

#include <type_traits>

#include "ga_device.h"
#include "ga_internal.h"
#include "ga_quant.h"
#include "ga_rope.h"

namespace ga {
namespace {

constexpr float kRescaleLog2 = 8.0f;

constexpr int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Waves per work-group: keeps the end-of-split LDS merge buffer at 32 KiB (four waves
// where that fits: with non-temporal loads four waves per CU already stream at the HBM
// rate measured for plain copies).
template <int D, int G>
constexpr int valu_nw_base() { return clampi(8192 / (G * D), 1, 4); }

template <int D, int G, int NW_>
struct ValuCfg {
  static constexpr int L = clampi(G * D / 64, 8, D / 8);  // lanes per key: acc <= 64..128 VGPRs
  static constexpr int DPL = D / L;                        // elements per lane per key
  static constexpr int NCH = DPL / 8;                      // 16-byte loads per lane per key
  static constexpr int GPW = 64 / L;                       // keys per wave per step
  static constexpr int NW = NW_;                           // waves per work-group
  static constexpr int NG = GPW * NW;                      // keys per work-group per step
  static_assert(NCH >= 1 && DPL % 8 == 0, "lane slice must be whole 16-byte chunks");
};

// G is the number of query rows a unit serves: the query heads of one KV head (one
// token), or with MULTI those heads for each of the Tc tokens of a chunk (row hh is
// token hh / Gh, head hh % Gh), every row masked at its own position.
// 32-bit word i of a 16- or 8-byte load chunk (i is a compile-time constant after
// unrolling).
__device__ __forceinline__ uint32_t chunk_word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t chunk_word(const uint2& v, int i) { return i == 0 ? v.x : v.y; }

// FP8: the cache holds e4m3 codes with one float32 scale per row (K and V each); a key's
// logit is scale_k * <q, codes> and its value weight p * scale_v multiplies the codes.
// ROPE: the rotary embedding fused with the append (single token, bf16 caches): q and the
// new K row rotate at new_pos[b] in the work-group (the same per-element function as the
// RoPE + append kernel, so the launch equals RoPE + append followed by decode, bit for bit).
template <int D, int G, int NW_, bool KV_SHARED, bool MULTI, bool FP8, bool ROPE = false>
__global__ void __launch_bounds__(NW_ * 64)
    decode_valu_kernel(DecodeArgs a) {
  static_assert(!ROPE || (!MULTI && !FP8), "RoPE is fused for single-token bf16 decode only");
  using C = ValuCfg<D, G, NW_>;
  constexpr int L = C::L, DPL = C::DPL, GPW = C::GPW, NW = C::NW;
  constexpr int ROW16 = D / 8;  // 16-byte chunks per bf16 row
  // A lane owns elements EPC * (c * L + j) + e (e < EPC) of each row, for its NCH load
  // chunks c: 8 bf16 or 16 fp8 codes per 16-byte chunk (8 codes in 8 bytes when a lane
  // owns only 8 elements).
  constexpr int EPC = FP8 ? (DPL >= 16 ? 16 : 8) : 8;
  constexpr int NCH = DPL / EPC;
  using Chunk = std::conditional_t<FP8 && EPC == 8, uint2, uint4>;
  constexpr int ROWC = (FP8 ? D : 2 * D) / (int)sizeof(Chunk);  // chunks per cache row
  static_assert(NCH >= 1 && DPL % EPC == 0, "lane slice must be whole load chunks");

  __shared__ __attribute__((aligned(16))) float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ __attribute__((aligned(16))) uint16_t s_rot[ROPE ? (G + 1) * D : 8];  // q, k_new

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / L;
  const int j = lane % L;

  const int S = a.n_split;
  int bid = blockIdx.x;
  const int split = bid % S;
  bid /= S;
  int chunk = 0;
  if constexpr (MULTI) {
    chunk = bid % a.n_chunks;
    bid /= a.n_chunks;
  }
  const int g = bid % a.Hkv;
  const int b = bid / a.Hkv;
  const int h0 = g * G;

  // Query row hh of this unit: its token, whether it exists, and its row index in q /
  // out / the partials ([B, Hq] rows, or [B, T, Hq] rows with MULTI).
  auto row_token = [&](int hh) { return MULTI ? chunk * a.Tc + hh / a.Gh : 0; };
  auto row_active = [&](int hh) { return !MULTI || row_token(hh) < a.T; };
  auto row_index = [&](int hh) -> size_t {
    if constexpr (!MULTI) return (size_t)b * a.Hq + h0 + hh;
    const int t = min(row_token(hh), a.T - 1);  // inactive rows alias the last token
    return ((size_t)b * a.T + t) * a.Hq + (size_t)g * a.Gh + hh % a.Gh;
  };

  // Fused append: split 0 of each unit moves the new row; its loads are issued here and
  // the stores happen after the key loop, so nothing waits on them.
  const int new_slot = appended_slot(a, b);
  AppendRow app;  // (bf16 rows; fp8 caches append their quantized rows below)
  app.load(a, b, g, new_slot, threadIdx.x, !FP8 && split == 0);
  // FP8 fused append (one token): wave 0 quantizes the new K row and wave 1 the new V row
  // (wave 0 both with one wave) exactly as the quantizing append does; their loads go out
  // here, ahead of the first K rows.
  constexpr bool APP8 = FP8 && !MULTI;
  constexpr int NROW8 = KV_SHARED ? 1 : 2;
  const bool app8 = APP8 && new_slot >= 0;  // the same in the whole work-group
  uint4 src8[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if constexpr (APP8) {
    if (app8 && lane < D / 8) {
      const size_t at = ((size_t)b * a.Hkv + g) * (D / 8) + lane;
#pragma unroll
      for (int rr = 0; rr < NROW8; ++rr)
        if (NW == 1 || wave == rr)
          src8[rr] = reinterpret_cast<const uint4*>(rr ? a.v_new : a.k_new)[at];
    }
  }
  // Query rows of this unit in this lane's element order, as packed bf16 pairs for the
  // dot2 products (fp8 keys are widened exactly to bf16 pairs first).  Loaded before the
  // context length is known (they do not depend on it), so the two latencies overlap.
  uint32_t qr[G][DPL / 2];  // element pairs (e, e + 1), e even, in lane order
  auto put_q = [&](int hh, int c, int h8, const uint4& v) {
    qr[hh][EPC * c / 2 + 4 * h8 + 0] = v.x;
    qr[hh][EPC * c / 2 + 4 * h8 + 1] = v.y;
    qr[hh][EPC * c / 2 + 4 * h8 + 2] = v.z;
    qr[hh][EPC * c / 2 + 4 * h8 + 3] = v.w;
  };
  // ROPE: the unit's G query rows and its new K row, unrotated, in 16-byte chunks (RPT
  // per thread), and the (cos, sin) of the rotate-half pairs (i, i + D/2) this thread turns
  // (NPR, i < rope_dim / 2), all
  // requested here, ahead of the first K rows; the rotation follows once those are out.
  constexpr int RCH = ROPE ? (G + 1) * D / 8 : 1;
  constexpr int RPT = (RCH + NW * 64 - 1) / (NW * 64);
  constexpr int NPR = ROPE ? (D / 2 + NW * 64 - 1) / (NW * 64) : 1;
  uint4 raw[RPT];
  double2 rcs[NPR];
  Chunk kfresh[ROPE ? NCH : 1];  // this lane's chunks of the rotated new K row
  if constexpr (!ROPE) {  // (with ROPE: from the rotated rows, once they are in LDS)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + row_index(hh) * D);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int h8 = 0; h8 < EPC / 8; ++h8) put_q(hh, c, h8, qp[(EPC / 8) * (c * L + j) + h8]);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < NPR; ++r) {
      const int i = threadIdx.x + r * NW * 64, half = a.rope_dim / 2;
      rcs[r] = i < half ? reinterpret_cast<const double2*>(a.rope_table)[(size_t)b * half + i]
                        : make_double2(1.0, 0.0);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int t = threadIdx.x + r * NW * 64;
      const int hh = t / (D / 8), c = t % (D / 8);
      const uint16_t* src =
          hh < G ? a.q + row_index(hh) * D : a.k_new + ((size_t)b * a.Hkv + g) * D;
      raw[r] = t < RCH ? *reinterpret_cast<const uint4*>(src + 8 * c) : make_uint4(0, 0, 0, 0);
    }
  }

  const size_t row0 = (size_t)(b * a.Hkv + g) * a.cap;
  const void* kmem = FP8 ? (const void*)a.k8 : (const void*)a.k;
  const void* vmem = FP8 ? (const void*)(KV_SHARED ? a.k8 : a.v8)
                         : (const void*)(KV_SHARED ? a.k : a.v);
  const Chunk* kbase = reinterpret_cast<const Chunk*>(kmem) + row0 * ROWC;
  const Chunk* vbase = reinterpret_cast<const Chunk*>(vmem) + row0 * ROWC;
  const float* kscale = FP8 ? a.k_scale + row0 : nullptr;
  const float* vscale = FP8 ? (KV_SHARED ? a.k_scale : a.v_scale) + row0 : nullptr;
  // fused append (bf16 caches): the appended token's rows, read in place of its slot
  const size_t unit = (size_t)b * a.Hkv + g;
  const Chunk* knew =
      !FP8 && a.new_pos ? reinterpret_cast<const Chunk*>(a.k_new) + unit * ROW16 : kbase;
  const Chunk* vnew =
      !FP8 && a.new_pos
          ? reinterpret_cast<const Chunk*>(KV_SHARED ? a.k_new : a.v_new) + unit * ROW16
          : vbase;

  // sc[0] / sc[1]: the key's K / V row scales (fp8 caches only).  The L lanes of a group
  // read L * sizeof(Chunk) >= 128 contiguous bytes per load, whole lines, so the cache
  // rows are loaded non-temporally (measured ~10% faster than cached loads here).
  static_assert(L * (int)sizeof(Chunk) >= 128, "a lane group reads whole 128-byte lines");
  auto load_rows = [&](Chunk(&kr)[NCH], Chunk(&vr)[NCH], float(&sc)[2], int slot, bool fresh) {
    const Chunk* kp = fresh ? knew : kbase + (size_t)slot * ROWC;
#pragma unroll
    for (int c = 0; c < NCH; ++c) kr[c] = stream_load(kp + c * L + j);
    if constexpr (!KV_SHARED) {
      const Chunk* vp = fresh ? vnew : vbase + (size_t)slot * ROWC;
#pragma unroll
      for (int c = 0; c < NCH; ++c) vr[c] = stream_load(vp + c * L + j);
    }
    if constexpr (FP8) {
      sc[0] = kscale[slot];
      sc[1] = KV_SHARED ? sc[0] : vscale[slot];
    }
  };

  // Single-token decode visits the keys of a range that starts at slot 0, or fills the
  // whole ring, in slot order: key i is slot i (any order of the same keys gives the
  // same result up to rounding).  The rows of a wave's first step (wave w takes step w)
  // then do not depend on the context length and are requested before it arrives; a lane
  // whose guess turns out wrong (another range, a key past the end, the appended slot)
  // reloads once the range is known.
  const int k_begin = split * a.split_keys;
  const int i_first = k_begin + wave * GPW + grp;
  Chunk ka[NCH], va[NCH];
  float ca[2] = {1.0f, 1.0f};
  if constexpr (!MULTI)
    load_rows(ka, va, ca, min(i_first, min(a.cap, k_begin + a.split_keys) - 1), false);

  if constexpr (ROPE) {
    // Rotate at the appended position: each thread takes rotate-half pairs (i, i + D/2)
    // and turns them in place in all G + 1 rows in LDS.  Every work-group of the unit does this; the
    // first split also writes the rotated q out and appends the rotated K row.
    const int half = a.rope_dim / 2;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int t = threadIdx.x + r * NW * 64;
      if (t < RCH) *reinterpret_cast<uint4*>(s_rot + 8 * t) = raw[r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NPR; ++r) {
      const int i = threadIdx.x + r * NW * 64;
      if (i < half) {
#pragma unroll
        for (int hh = 0; hh <= G; ++hh) {
          uint16_t* row = s_rot + hh * D;
          const uint16_t x0 = row[i], x1 = row[i + D / 2];
          row[i] = rope_first(x0, x1, rcs[r].x, rcs[r].y);
          row[i + D / 2] = rope_second(x0, x1, rcs[r].x, rcs[r].y);
        }
      }
    }
    __syncthreads();
    if (split == 0)
      for (int e = threadIdx.x; e < G * D; e += NW * 64)
        a.q_rot_out[row_index(e / D) * D + e % D] = s_rot[e];
    if (app.on) app.k = *reinterpret_cast<const AppendRow::u32x4*>(s_rot + G * D + 8 * threadIdx.x);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      kfresh[c] = *reinterpret_cast<const Chunk*>(s_rot + G * D + (c * L + j) * 8);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4* qp = reinterpret_cast<const uint4*>(s_rot + hh * D);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int h8 = 0; h8 < EPC / 8; ++h8) put_q(hh, c, h8, qp[(EPC / 8) * (c * L + j) + h8]);
      }
    }
  }
  // FP8 fused append: the quantized rows into LDS, this lane's chunks of them and their
  // scales into registers (they replace the appended key's loaded rows where the loop
  // consumes them), and the first split stores them into the slot.  Every reader of that
  // slot in this launch is a work-group of this unit and takes the registers, so when the
  // store lands does not matter.
  __shared__ __attribute__((aligned(16))) uint8_t s_c8[APP8 ? 2 * D : 16];
  __shared__ float s_c8s[2];
  Chunk kf8[APP8 ? NCH : 1], vf8[APP8 ? NCH : 1];
  float sf8[2] = {1.0f, 1.0f};
  if constexpr (APP8) {
    if (app8) {
      if (wave < NROW8) {
        const size_t row8 = ((size_t)b * a.Hkv + g) * a.cap + new_slot;
#pragma unroll
        for (int rr = 0; rr < NROW8; ++rr) {
          if (NW > 1 && wave != rr) continue;  // (the same in the whole wave)
          float s8;
          const uint2 c8 = quantize_row_e4m3(src8[rr], lane < D / 8, &s8);
          if (lane < D / 8) {
            *reinterpret_cast<uint2*>(s_c8 + rr * D + 8 * lane) = c8;
            if (split == 0) reinterpret_cast<uint2*>((rr ? a.v8_dst : a.k8_dst) + row8 * D)[lane] = c8;
          }
          if (lane == 0) {
            s_c8s[rr] = s8;
            if (split == 0) (rr ? a.vs_dst : a.ks_dst)[row8] = s8;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        kf8[c] = *reinterpret_cast<const Chunk*>(s_c8 + EPC * (c * L + j));
        if constexpr (!KV_SHARED) vf8[c] = *reinterpret_cast<const Chunk*>(s_c8 + D + EPC * (c * L + j));
      }
      sf8[0] = s_c8s[0];
      sf8[1] = KV_SHARED ? sf8[0] : s_c8s[1];
    }
  }

  const RowRange r = unit_range(a, b, chunk);
  const int k_end = min(r.n, k_begin + a.split_keys);
  if (k_begin >= k_end) {
    if (S == 1) {  // the only split of an empty unit: the output is 0
      for (int idx = threadIdx.x; idx < G * D; idx += NW * 64)
        if (row_active(idx / D)) a.out[row_index(idx / D) * D + idx % D] = 0.0f;
    }
    app.store(a);
    return;  // with S > 1 the merge never reads splits past the unit's end
  }
  __shared__ int s_next;  // handed-out wave-steps past the first NW
  if (threadIdx.x == 0) s_next = 0;
  // key i of the range sits in slot key_slot(slot_base, i): position order, or slot order
  // (slot_base 0) for single-token decode over a full ring; several tokens keep position
  // order (their masks are by position)
  const int slot_base = (!MULTI && r.n == a.cap) ? 0 : r.slot_lo;

  // MULTI: each row's own valid positions [row_lo, row_hi] (empty: lo > hi).
  int row_lo[MULTI ? G : 1], row_hi[MULTI ? G : 1];
  if constexpr (MULTI) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      row_lo[hh] = 1;
      row_hi[hh] = 0;
      if (row_active(hh)) {
        const RowRange rr = row_range(a.ctx[b], a.q_pos[b] + row_token(hh), a.window, a.kind,
                                      a.cap, a.max_keys);
        if (rr.n > 0) {
          row_lo[hh] = rr.lo;
          row_hi[hh] = rr.hi;
        }
      }
    }
  }


  float acc[G][DPL];
  float m[G], l[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;
  }

  // Wave-step s covers keys k_begin + s * GPW + grp (one per lane group).  Wave w's first
  // step is w, so its first rows are requested before any barrier; later steps are
  // handed out as waves ask for them (an LDS counter), so waves that the SIMD arbiter
  // serves less still finish together with the others.  In deterministic mode the order
  // is static (wave w takes w, w + NW, ...), which fixes the summation order.
  const int n_wsteps = (k_end - k_begin + GPW - 1) / GPW;
  const float scale = a.scale;
  const float softcap = a.softcap, inv_softcap = a.inv_softcap;
  int taken = 0;
  auto grab = [&]() -> int {
    if (a.deterministic || taken == 0) return wave + NW * (taken++);
    int s = 0;
    if (lane == 0) s = atomicAdd(&s_next, 1);
    return NW + __builtin_amdgcn_readfirstlane(s);
  };

  auto load = [&](Chunk(&kr)[NCH], Chunk(&vr)[NCH], float(&sc)[2], int step) {
    const int i = k_begin + step * GPW + grp;
    const int ic = i < k_end ? i : k_end - 1;  // past the end: re-read a valid row
    const int slot = key_slot(slot_base, ic, a.cap);
    load_rows(kr, vr, sc, slot, !FP8 && slot == new_slot);
  };

  // e4m3 codes of one chunk -> bf16 pairs (v_cvt_scalef32_pk_bf16_fp8 with scale 1,
  // exact: checked bit for bit on all 256 codes), for the dot2 products with q
  auto widen_fp8_bf16 = [&](const Chunk& ch, uint32_t* out) {
#pragma unroll
    for (int w = 0; w < EPC / 4; ++w) {
      const int word = (int)chunk_word(ch, w);
      out[2 * w + 0] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
      out[2 * w + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
    }
  };
  // e4m3 codes of one chunk -> float32 values (v_cvt_pk_f32_fp8, exact), for P.V
  auto widen_fp8 = [&](const Chunk& ch, float* out) {
    typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < EPC / 4; ++w) {
      const int word = (int)chunk_word(ch, w);
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      out[4 * w + 0] = lo.x;
      out[4 * w + 1] = lo.y;
      out[4 * w + 2] = hi.x;
      out[4 * w + 3] = hi.y;
    }
  };

  auto compute = [&](const Chunk(&kr)[NCH], const Chunk(&vr)[NCH], const float(&sc)[2],
                     int step) {
    const int i = k_begin + step * GPW + grp;
    const bool valid = i < k_end;
    // The key rows; with ROPE the appended key (its slot's load read the unrotated k_new)
    // takes the rotated row held in registers, selected here where the loaded rows are
    // consumed, so the loads themselves stay unconditional.
    // (FP8 appending: the appended key's quantized rows and scales likewise.)
    Chunk kx[NCH], vx[NCH];
    float scx[2] = {sc[0], sc[1]};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      kx[c] = kr[c];
      vx[c] = vr[c];
    }
    if constexpr (ROPE) {
      if (key_slot(slot_base, valid ? i : k_end - 1, a.cap) == new_slot) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) kx[c] = kfresh[c];
      }
    }
    if constexpr (APP8) {
      if (app8 && key_slot(slot_base, valid ? i : k_end - 1, a.cap) == new_slot) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          kx[c] = kf8[c];
          if constexpr (!KV_SHARED) vx[c] = vf8[c];
        }
        scx[0] = sf8[0];
        scx[1] = sf8[1];
      }
    }
    const int pos = r.lo + i;  // absolute position of the key (MULTI masks)
    float s[G];
    if constexpr (FP8) {
      uint32_t kb[DPL / 2];
#pragma unroll
      for (int c = 0; c < NCH; ++c) widen_fp8_bf16(kx[c], &kb[EPC * c / 2]);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int e2 = 0; e2 < DPL / 2; e2 += 2) {
          d0 = dot2_bf16(qr[hh][e2], kb[e2], d0);
          d1 = dot2_bf16(qr[hh][e2 + 1], kb[e2 + 1], d1);
        }
        s[hh] = group_sum<L>(d0 + d1) * scx[0];
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          d0 = dot2_bf16(qr[hh][4 * c + 0], chunk_word(kx[c], 0), d0);
          d1 = dot2_bf16(qr[hh][4 * c + 1], chunk_word(kx[c], 1), d1);
          d0 = dot2_bf16(qr[hh][4 * c + 2], chunk_word(kx[c], 2), d0);
          d1 = dot2_bf16(qr[hh][4 * c + 3], chunk_word(kx[c], 3), d1);
        }
        s[hh] = group_sum<L>(d0 + d1);
      }
    }
    float p[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      bool vh = valid;
      if constexpr (MULTI) vh = vh && pos >= row_lo[hh] && pos <= row_hi[hh];
      float x = s[hh] * scale;
      if (softcap > 0.0f) x = softcap_tanh(x, softcap, inv_softcap);
      x = vh ? x * kLog2e : -INFINITY;
      if (x > m[hh] + kRescaleLog2) {
        const float f = exp2_fast(m[hh] - x);  // 0 on the first key (m = -inf)
        l[hh] *= f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[hh][e] *= f;
        m[hh] = x;
      }
      p[hh] = vh ? exp2_fast(x - m[hh]) : 0.0f;
      l[hh] += p[hh];
    }
    const Chunk(&vv)[NCH] = KV_SHARED ? kx : vx;
    if constexpr (FP8) {
      float pv[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pv[hh] = p[hh] * scx[1];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float vf[EPC];
        widen_fp8(vv[c], vf);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            acc[hh][EPC * c + e] = fmaf(pv[hh], vf[e], acc[hh][EPC * c + e]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = chunk_word(vv[c], t);
          const float lo = bf16_lo(w), hi = bf16_hi(w);
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            acc[hh][8 * c + 2 * t] = fmaf(p[hh], lo, acc[hh][8 * c + 2 * t]);
            acc[hh][8 * c + 2 * t + 1] = fmaf(p[hh], hi, acc[hh][8 * c + 2 * t + 1]);
          }
        }
      }
    }
  };

  // Two register buffers: the next step's rows are in flight while a step computes.  The
  // loads are unconditional (past the end they re-read the last valid row) and the loop
  // body is straight-line with its test at the bottom, so every path into the loop
  // header carries the same outstanding loads (buffer a only) and the compiler keeps
  // partial vmcnt waits instead of draining the prefetch.  Grabs are increasing per wave,
  // so sa < sb < n_wsteps inside the loop.
  Chunk kb[NCH], vb[NCH];
  float cb[2] = {1.0f, 1.0f};
  int sa = grab();  // = wave
  if constexpr (MULTI) {
    load(ka, va, ca, sa);
  } else {
    // the guessed rows stand unless the range is not in slot order, the key is past the
    // end (the guess may be a slot never written), or the slot is the appended one
    const int slot = key_slot(slot_base, min(i_first, k_end - 1), a.cap);
    if (slot_base != 0 || i_first >= k_end || (!FP8 && slot == new_slot)) load(ka, va, ca, sa);
  }
  __syncthreads();  // s_next is set before any wave asks for a handed-out step
  int sb = grab();
  while (sb < n_wsteps) {
    load(kb, vb, cb, sb);
    compute(ka, va, ca, sa);
    sa = grab();
    load(ka, va, ca, sa);
    compute(kb, vb, cb, sb);
    sb = grab();
  }
  if (sa < n_wsteps) compute(ka, va, ca, sa);
  app.store(a);

  // Merge the GPW groups of this wave (lanes j, j + L, j + 2L, ... hold the same
  // elements).  Each group first rescales to the wave's common max M, so that merging is
  // a plain sum.  At the lane offsets 32 and 16 the sum is a reduce-scatter: one
  // v_permlane32/16_swap of the value pair (x_i, x_{i + n/2}) hands the lower lane both
  // copies of x_i and the upper lane both copies of x_{i + n/2}, so each level halves the
  // values a lane holds (while at least 8 remain); the other levels are butterflies
  // (both lanes keep the full sum).  Both lanes of a pair add the same two numbers in
  // the same order, so the result does not depend on which lane computes it.
  constexpr int NV = G * DPL;  // values per lane: acc flattened as [hh][e]
  constexpr bool RS32 = L <= 32 && NV / 2 >= 8;
  constexpr int NV1 = RS32 ? NV / 2 : NV;
  constexpr bool RS16 = L <= 16 && NV1 / 2 >= 8;
  constexpr int NV2 = RS16 ? NV1 / 2 : NV1;
  static_assert(NV2 % 4 == 0, "float4 runs of the accumulator");
  float M[G], Lw[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    M[hh] = m[hh];
    if constexpr (L <= 8) M[hh] = fmaxf(M[hh], xor_lane<8>(M[hh], lane));
    if constexpr (L <= 16) M[hh] = fmaxf(M[hh], xor_lane<16>(M[hh], lane));
    if constexpr (L <= 32) M[hh] = fmaxf(M[hh], xor_lane<32>(M[hh], lane));
  }
  float vf[NV];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float f = m[hh] == -INFINITY ? 0.0f : exp2_fast(m[hh] - M[hh]);
    Lw[hh] = l[hh] * f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) vf[hh * DPL + e] = acc[hh][e] * f;
    float lo, hi;
    if constexpr (L <= 8) Lw[hh] += dpp<kDppRowRor8>(Lw[hh]);
    if constexpr (L <= 16) {
      lane_pair16(Lw[hh], lo, hi);
      Lw[hh] = lo + hi;
    }
    if constexpr (L <= 32) {
      lane_pair32(Lw[hh], lo, hi);
      Lw[hh] = lo + hi;
    }
  }
  if constexpr (L <= 32) {
#pragma unroll
    for (int i = 0; i < NV1; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(
          __float_as_int(vf[i]), __float_as_int(vf[RS32 ? i + NV / 2 : i]), false, false);
      vf[i] = __int_as_float(r[0]) + __int_as_float(r[1]);
    }
  }
  if constexpr (L <= 16) {
#pragma unroll
    for (int i = 0; i < NV2; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(
          __float_as_int(vf[i]), __float_as_int(vf[RS16 ? i + NV1 / 2 : i]), false, false);
      vf[i] = __int_as_float(r[0]) + __int_as_float(r[1]);
    }
  }
  if constexpr (L <= 8) {
#pragma unroll
    for (int i = 0; i < NV2; ++i) vf[i] += dpp<kDppRowRor8>(vf[i]);
  }

  // Merge the waves through LDS, then write the output or this split's partial.  Lane
  // value i is element base + i of the flattened [hh][e] accumulator; of the lanes that
  // a butterfly level left identical, the one with that lane bit clear writes.
  const int base = (RS32 ? ((lane >> 5) & 1) * (NV / 2) : 0) +
                   (RS16 ? ((lane >> 4) & 1) * (NV1 / 2) : 0);
  const int dup_bits = (L <= 8 ? 8 : 0) | (L <= 16 && !RS16 ? 16 : 0) |
                       (L <= 32 && !RS32 ? 32 : 0);
  if ((lane & dup_bits) == 0) {
#pragma unroll
    for (int i = 0; i < NV2; i += 4) {
      const int f = base + i;
      const int hh = f / DPL, e = f % DPL;
      float* dst = &s_acc[wave][hh][EPC * ((e / EPC) * L + j) + e % EPC];
      *reinterpret_cast<float4*>(dst) = make_float4(vf[i], vf[i + 1], vf[i + 2], vf[i + 3]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_m[wave][hh] = M[hh];
      s_l[wave][hh] = Lw[hh];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int hh = idx / D, d = idx % D;
    if (!row_active(hh)) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hh]);
    float Lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = s_m[w][hh] == -INFINITY ? 0.0f : exp2_fast(s_m[w][hh] - M);
      Lsum += s_l[w][hh] * f;
      o += s_acc[w][hh][d] * f;
    }
    const size_t bh = row_index(hh);
    if (S == 1) {
      a.out[bh * D + d] = Lsum > 0.0f ? o / Lsum : 0.0f;
    } else {
      a.part_acc[(bh * S + split) * D + d] = o;
      if (d == 0) {
        a.part_ml[(bh * S + split) * 2 + 0] = M;
        a.part_ml[(bh * S + split) * 2 + 1] = Lsum;
      }
    }
  }
}

template <int D, int G, int NW>
hipError_t launch_dgw(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  const long long blocks = (long long)a.B * a.Hkv * a.n_chunks * a.n_split;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(NW * 64);
  const bool multi = a.T > 1;
  // K = V, several tokens, fp8 cache: one instantiation per combination
#define GA_VALU_LAUNCH(KV, MU, F8)                                                             \
  hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, KV, MU, F8>), grid, block, 0, stream, a)
#define GA_VALU_LAUNCH_ROPE(KV)                                                                \
  hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, KV, false, false, true>), grid, block, 0,    \
                     stream, a)
  if (a.rope) {  // single token, bf16 caches (the plan checks)
    if (multi || a.fp8) return hipErrorInvalidValue;
    if (k_eq_v) GA_VALU_LAUNCH_ROPE(true); else GA_VALU_LAUNCH_ROPE(false);
  } else if (a.fp8) {
    if (multi) {
      if (k_eq_v) GA_VALU_LAUNCH(true, true, true); else GA_VALU_LAUNCH(false, true, true);
    } else {
      if (k_eq_v) GA_VALU_LAUNCH(true, false, true); else GA_VALU_LAUNCH(false, false, true);
    }
  } else {
    if (multi) {
      if (k_eq_v) GA_VALU_LAUNCH(true, true, false); else GA_VALU_LAUNCH(false, true, false);
    } else {
      if (k_eq_v) GA_VALU_LAUNCH(true, false, false); else GA_VALU_LAUNCH(false, false, false);
    }
  }
#undef GA_VALU_LAUNCH
#undef GA_VALU_LAUNCH_ROPE
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  return launch_dgw<D, G, valu_nw_base<D, G>()>(a, k_eq_v, stream);
}

}  // namespace

// All instantiations for one head dim (explicitly instantiated per head dim).
template <int D>
hipError_t valu_launch_d(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  switch (a.Gh * a.Tc) {  // query rows per unit
    case 1: return launch_dg<D, 1>(a, k_eq_v, stream);
    case 2: return launch_dg<D, 2>(a, k_eq_v, stream);
    case 4: return launch_dg<D, 4>(a, k_eq_v, stream);
    case 8: return launch_dg<D, 8>(a, k_eq_v, stream);
    case 16: return launch_dg<D, 16>(a, k_eq_v, stream);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace ga
