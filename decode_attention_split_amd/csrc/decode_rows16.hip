// decode_rows16.hip -- matrix-core split decode for 16 query rows per KV head: several
// query tokens per sequence (speculative verification, chunked prefill) on the same
// caches, each row masked at its own position.
//
// Why matrix cores: with 16 query rows on one KV head every cached byte feeds about 16
// flops (q.k and p.v for each row), so the vector kernel, which reduces every row's dot
// product across the lanes of a key, runs out of ALU long before HBM.  Here one
// work-group of four waves (two at head_dim 512) owns one split (a run of keys of one
// unit = batch row, KV head, chunk of tokens); its waves take the split's 16-key tiles in
// turn (wave w: tiles w, w + 4, ...), each with its own softmax state.  Per tile:
//   the tile's K and V rows are loaded with every instruction covering whole rows (whole
//     128-byte lines, non-temporal), then written to the wave's LDS tiles in natural d order
//     (fp8 codes widened exactly to bf16 on the way);
//   S^T[16 keys][16 rows] = K[16][D] . Q^T[D][16]: D / 32 v_mfma_f32_16x16x32_bf16, the
//     K operand read back from the K tile (lane: key l16, d = 8 lg + 32 j + 0..7), Q^T read
//     from LDS (shared by the waves) in the same d order;
//   S^T leaves lane l holding row l16 for keys 4 lg + 0..3, which is exactly the B operand
//     of the P.V product, so the softmax works in place (row max / sum over the four lane
//     groups) and P goes to the matrix cores as bf16 hi + lo parts (~16 mantissa bits);
//   the V tile comes back transposed with ds_read_b64_tr_b16 as the A operand of
//     O^T[D][16] += V^T[D][16 keys] . P^T[16 keys][16 rows]: D / 16
//     v_mfma_f32_16x16x32_bf16, each with the tile's keys in both halves of the k slots
//     against P's hi and lo parts (with K = V one tile serves both products).
// One register buffer each for K and V, refilled as soon as the tile's rows are in LDS
// (eight waves per CU hide the latency).  Loading each key's row in 16-byte pieces straight
// into the K operand (lane l16 = key) reads half lines per instruction and streamed at
// 5.45 TB/s on the spec-decode layer; whole-row loads stream faster.  At the end the waves merge through LDS, so a
// split is one partial: with one split per unit (batches that fill the chip) the output is
// written directly and no merge kernel runs; otherwise each split leaves (m, l, acc) for
// the log-sum-exp merge.  (A merge by the last split to arrive would need a device-scope
// release per work-group, which on this chip writes back the L2 and costs more than the
// separate merge.)  Softmax in log2 units, lazily rescaled (max raised only past +8);
// masked keys weigh exactly zero.
//
// Definition followed: the same single-token definition per query token ("Gemma support"
// pull request, Summary and Performance; "Gemma 4 12B (unified multimodal)" record: the
// window of exactly w entries, spec decode with sliding windows in item (2)); key ranges
// from ga::unit_range / ga::row_range, as in every other kernel.
#include "ga_device.h"
#include "ga_internal.h"
#include "ga_mfma.h"

namespace ga {
namespace {

constexpr float kRescaleLog2R16 = 8.0f;
#ifndef GA_ROWS16_BUFS
#define GA_ROWS16_BUFS 1
#endif

template <int D>
constexpr int rows16_waves() { return D == 512 ? 2 : 4; }

template <int D, bool KV_SHARED, bool FP8>
__global__ void __launch_bounds__(64 * rows16_waves<D>()) decode_rows16_kernel(DecodeArgs a) {
  constexpr int NW = rows16_waves<D>();  // waves per work-group, one split between them
  constexpr int NJ = D / 32;             // 16-byte K chunks per lane = QK products per tile
  constexpr int NDB = D / 16;            // 16-wide head_dim blocks of the output
  constexpr int ROWB = D * 2 + 32;       // LDS bytes per key row (padding spreads the banks)
  constexpr int QROWB = D * 2 + 16;      // LDS bytes per query row
  constexpr int Q_BYTES = 16 * QROWB;
  constexpr int TILE_BYTES = 16 * ROWB;
  constexpr int NTILES = KV_SHARED ? 1 : 2;                       // K (and V) tile per wave
  constexpr int LOOP_BYTES = Q_BYTES + NW * NTILES * TILE_BYTES;  // Q rows + the tiles
  constexpr int ACC_BYTES = NW * 16 * D * 4;             // the waves' accumulators (end)
  __shared__ __attribute__((aligned(16))) char s_mem[LOOP_BYTES > ACC_BYTES ? LOOP_BYTES
                                                                            : ACC_BYTES];
  __shared__ float s_ml[NW][16][2];
  __shared__ __attribute__((aligned(16))) float s_scl[NW][2][16];  // fp8: K, V row scales

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  const int S = a.n_split;
  int bid = blockIdx.x;
  const int split = bid % S;
  bid /= S;
  const int chunk = bid % a.n_chunks;
  bid /= a.n_chunks;
  const int g = bid % a.Hkv;
  const int b = bid / a.Hkv;

  // query row rr of the unit: token chunk * Tc + rr / Gh, head g * Gh + rr % Gh
  auto row_token = [&](int rr) { return chunk * a.Tc + rr / a.Gh; };
  auto row_index = [&](int rr) -> size_t {
    const int t = min(row_token(rr), a.T - 1);  // inactive rows alias the last token
    return ((size_t)b * a.T + t) * a.Hq + (size_t)g * a.Gh + rr % a.Gh;
  };
  const bool row_on = row_token(l16) < a.T;  // this lane's row is l16
  const size_t row = row_index(l16);

  const int ctx_b = a.ctx[b], qpos_b = a.q_pos[b];  // (read once: the row ranges below too)
  const RowRange r = unit_range_of(a, ctx_b, qpos_b, chunk);
  const int k_begin = split * a.split_keys;
  const int k_end = min(r.n, k_begin + a.split_keys);
  if (k_begin >= k_end) {
    // the only split of an empty unit writes its zero output; with several splits the
    // merge writes it
    if (S == 1 && row_on && wave == 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<floatx4_t*>(a.out + row * D + 16 * db + 4 * lg) =
            floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  // the row's own valid positions (empty: lo > hi)
  int row_lo = 1, row_hi = 0;
  if (row_on) {
    const RowRange rr = row_range(ctx_b, qpos_b + row_token(l16), a.window, a.kind, a.cap,
                                  a.max_keys);
    if (rr.n > 0) {
      row_lo = rr.lo;
      row_hi = rr.hi;
    }
  }

  // Q^T operand (row l16, d = 8 lg + 32 j + 0..7) parked in LDS (the waves share it) and
  // read per product, which keeps the registers for the K / V tiles in flight and the
  // accumulators
  char* s_q = s_mem;
  // this wave's chunks j = wave, wave + NW, ... requested together; at head_dim <= 256 they
  // go to LDS only once the first tiles are requested too (so those do not wait for them)
  constexpr int QJ = (NJ + NW - 1) / NW;
  constexpr bool Q_LATE = D <= 256;
  u32x4_t qv[QJ];
  {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q + row * D);
#pragma unroll
    for (int i = 0; i < QJ; ++i) qv[i] = qp[4 * min(wave + NW * i, NJ - 1) + lg];
  }
  __builtin_amdgcn_sched_barrier(0);  // (issued before the tiles' loads, waited for first)
  auto put_q = [&]() {
#pragma unroll
    for (int i = 0; i < QJ; ++i) {
      const int j = wave + NW * i;
      if (j < NJ) *reinterpret_cast<u32x4_t*>(s_q + l16 * QROWB + (lg + 4 * j) * 16) = qv[i];
    }
  };
  if constexpr (!Q_LATE) put_q();
  const char* q_lds = s_q + l16 * QROWB + lg * 16;
  char* ktile = s_mem + Q_BYTES + wave * NTILES * TILE_BYTES;  // this wave's K tile
  char* tile = ktile + (NTILES - 1) * TILE_BYTES;              // and V tile (K = V: the same)
  const size_t row0 = (size_t)(b * a.Hkv + g) * a.cap;
  // (native 4 x u32 vectors: arrays of them stay in registers)
  // Cache rows in 16-byte chunks: bf16 rows hold D / 8, fp8 rows D / 16 (16 codes each).
  // A load instruction covers KPI whole rows: lane reads chunk lane % ROW16 of key
  // lane / ROW16 + KPI j of the tile (NL loads per lane and tile).
  constexpr int ROW16 = FP8 ? D / 16 : D / 8;
  static_assert(64 % ROW16 == 0, "rows per load instruction");
  constexpr int KPI = 64 / ROW16;
  constexpr int NL = 16 / KPI;
  const int lrow = lane / ROW16, lcol = lane % ROW16;
  const void* kmem = FP8 ? (const void*)a.k8 : (const void*)a.k;
  const void* vmem = FP8 ? (const void*)(KV_SHARED ? a.k8 : a.v8)
                         : (const void*)(KV_SHARED ? a.k : a.v);
  const u32x4_t* kbase = reinterpret_cast<const u32x4_t*>(kmem) + row0 * ROW16;
  const u32x4_t* vbase = reinterpret_cast<const u32x4_t*>(vmem) + row0 * ROW16;
  const float* kscale = FP8 ? a.k_scale + row0 : nullptr;
  const float* vscale = FP8 ? (KV_SHARED ? a.k_scale : a.v_scale) + row0 : nullptr;

  floatx4_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;

  // tiles of 16 keys; wave w takes tiles w, w + NW, ... of the split (a fixed order)
  const int nt = (k_end - k_begin + 15) / 16;
  // one tile's registers: its K (and V) row pieces, and (fp8) the row scales of key l16
  struct Regs {
    u32x4_t k[NL], v[KV_SHARED ? 1 : NL];
    float ks, vs;
  };
  // slot of key i of the split (past the end: the last valid key, re-read)
  auto slot_at = [&](int i) { return key_slot(r, i < k_end ? i : k_end - 1, a.cap); };
  auto load = [&](Regs& rg, int t) {
    const int k0 = k_begin + 16 * t;
#pragma unroll
    for (int j = 0; j < NL; ++j)
      rg.k[j] = stream_load(kbase + (size_t)slot_at(k0 + lrow + KPI * j) * ROW16 + lcol);
    if constexpr (!KV_SHARED) {
#pragma unroll
      for (int j = 0; j < NL; ++j)
        rg.v[j] = stream_load(vbase + (size_t)slot_at(k0 + lrow + KPI * j) * ROW16 + lcol);
    }
    if constexpr (FP8) {
      const int slot = slot_at(k0 + l16);
      rg.ks = kscale[slot];
      rg.vs = KV_SHARED ? rg.ks : vscale[slot];
    }
  };
  // a loaded row piece to its LDS tile (fp8 codes widened exactly to bf16)
  auto put = [&](char* dst, int j, const u32x4_t& x) {
    char* row = dst + (lrow + KPI * j) * ROWB;
    if constexpr (FP8) {
      *reinterpret_cast<uint4*>(row + lcol * 32) = e4m3x8_to_bf16x8(x.x, x.y);
      *reinterpret_cast<uint4*>(row + lcol * 32 + 16) = e4m3x8_to_bf16x8(x.z, x.w);
    } else {
      *reinterpret_cast<u32x4_t*>(row + lcol * 16) = x;
    }
  };
  // NB tiles in flight per wave: wave w's i-th tile t = w + NW i sits in regs[i % NB]
  constexpr int NB = GA_ROWS16_BUFS;
  Regs regs[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) load(regs[i], min(wave + NW * i, nt - 1));
  if constexpr (Q_LATE) put_q();
  __syncthreads();  // the Q rows are in LDS

  auto step = [&](Regs& rg, int t) {
    const int k0 = k_begin + 16 * t;
    // the tile's rows to LDS, then the registers refill with the wave's tile NB ahead
#pragma unroll
    for (int j = 0; j < NL; ++j) put(ktile, j, rg.k[j]);
    if constexpr (!KV_SHARED) {
#pragma unroll
      for (int j = 0; j < NL; ++j) put(tile, j, rg.v[j]);
    }
    if constexpr (FP8) {
      if (lg == 0) {  // the tile's row scales, read back per key 4 lg + i after the sync
        s_scl[wave][0][l16] = rg.ks;
        s_scl[wave][1][l16] = rg.vs;
      }
    }
    load(rg, t + NB * NW < nt ? t + NB * NW : t);
    wave_lds_sync();  // the tile's LDS writes before the reads below
    // S^T for the tile: K rows from the K tile (key l16, d = 32 j + 8 lg + 0..7)
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
    {
      const char* kq_lds = ktile + l16 * ROWB + lg * 16;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        s = mfma_k32(*reinterpret_cast<const u32x4_t*>(kq_lds + j * 64),
                     *reinterpret_cast<const u32x4_t*>(q_lds + j * 64), s);
    }

    // softmax: lane holds row l16, keys k0 + 4 lg + i
    float kq[4] = {1.0f, 1.0f, 1.0f, 1.0f}, vq[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (FP8) {  // the row scales of keys 4 lg + 0..3
      const float4 k4 = *reinterpret_cast<const float4*>(&s_scl[wave][0][4 * lg]);
      const float4 v4 = *reinterpret_cast<const float4*>(&s_scl[wave][1][4 * lg]);
      kq[0] = k4.x; kq[1] = k4.y; kq[2] = k4.z; kq[3] = k4.w;
      vq[0] = v4.x; vq[1] = v4.y; vq[2] = v4.z; vq[3] = v4.w;
    }
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + 4 * lg + i;
      const int pos = r.lo + key;
      float v = s[i] * kq[i] * a.scale;  // fp8: the key's row scale
      if (a.softcap > 0.0f) v = softcap_tanh(v, a.softcap, a.inv_softcap);
      const bool ok = key < k_end && pos >= row_lo && pos <= row_hi;
      x[i] = ok ? v * kLog2e : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = rows_max(mx);  // over the 16 keys of the tile (four lane groups)
    // rescale when some row's maximum grew past its reference: a branch on the whole
    // wave (rows that did not grow multiply by exactly 1), so the tiles that need none
    // leave the accumulators alone (a per-row condition is turned into selects, which
    // multiply and write back every accumulator register on every tile)
    const bool grow = mx > m + kRescaleLog2R16;
    if (__ballot(grow) != 0) {
      const float f = grow ? exp2_fast(m - mx) : 1.0f;  // 0 while m = -inf
      l *= f;
#pragma unroll
      for (int i = 0; i < NDB; ++i) acc[i] *= f;
      m = grow ? mx : m;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = x[i] == -INFINITY ? 0.0f : exp2_fast(x[i] - m);
      l += p[i];
      p[i] *= vq[i];  // fp8: the value row's scale (1 for bf16)
    }
    const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
    const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const short4_t ph = __builtin_bit_cast(short4_t, make_uint2(h01, h23));
    const short4_t pl = __builtin_bit_cast(short4_t, make_uint2(l01, l23));
    const char* rd = tile + (4 * lg + (l16 >> 2)) * ROWB + (l16 & 3) * 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const short4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(rd + db * 32));
      // both halves of the k slots hold the tile's keys: P's hi part against the first,
      // its lo part against the second (one 16x16x32 product; the 16x16x16 form costs as
      // many cycles on gfx950)
      acc[db] = mfma_k32(cat4(va, va), cat4(ph, pl), acc[db]);
    }
    wave_lds_sync();  // the tile's transposed reads stay before the next tile's writes
  };
  for (int t = wave; t < nt; t += NB * NW) {
    step(regs[0], t);
#pragma unroll
    for (int i = 1; i < NB; ++i)
      if (t + NW * i < nt) step(regs[i], t + NW * i);
  }

  // Merge the waves: each leaves (m, l) per row and acc (row l16, d = 16 db + 4 lg + i)
  // in LDS (over the Q rows and V tiles, no longer read), then every thread combines
  // float4 runs of the 16 rows: o = sum_w 2^(m_w - M) acc_w, L = sum_w 2^(m_w - M) l_w.
  l = rows_sum(l);
  __syncthreads();
  float* s_acc = reinterpret_cast<float*>(s_mem);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<floatx4_t*>(s_acc + (wave * 16 + l16) * D + 16 * db + 4 * lg) = acc[db];
  if (lg == 0) {
    s_ml[wave][l16][0] = m;
    s_ml[wave][l16][1] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < 16 * (D / 4); idx += NW * 64) {
    const int rr = idx / (D / 4), d = 4 * (idx % (D / 4));
    if (row_token(rr) >= a.T) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][rr][0]);
    float L = 0.0f;
    floatx4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_ml[w][rr][0];
      const float f = mw == -INFINITY ? 0.0f : exp2_fast(mw - M);
      L += s_ml[w][rr][1] * f;
      o += *reinterpret_cast<const floatx4_t*>(s_acc + (w * 16 + rr) * D + d) * f;
    }
    const size_t bh = row_index(rr);
    if (S == 1) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      *reinterpret_cast<floatx4_t*>(a.out + bh * D + d) = o * inv;
    } else {
      const size_t ps = bh * S + split;
      *reinterpret_cast<floatx4_t*>(a.part_acc + ps * D + d) = o;
      if (d == 0) {
        a.part_ml[ps * 2 + 0] = M;
        a.part_ml[ps * 2 + 1] = L;
      }
    }
  }
}


}  // namespace

int decode_rows16_waves(int D) { return D == 512 ? rows16_waves<512>() : rows16_waves<256>(); }

bool decode_rows16_supported(int D, bool k_eq_v) {
  return D == 128 || D == 256 || (D == 512 && k_eq_v);
}

hipError_t decode_rows16_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  const long long blocks = (long long)a.B * a.Hkv * a.n_chunks * a.n_split;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(64 * decode_rows16_waves(a.D));
#define GA_ROWS16_LAUNCH(DD, KV)                                                           \
  do {                                                                                     \
    if (a.fp8)                                                                             \
      hipLaunchKernelGGL((decode_rows16_kernel<DD, KV, true>), grid, block, 0, stream, a);  \
    else                                                                                   \
      hipLaunchKernelGGL((decode_rows16_kernel<DD, KV, false>), grid, block, 0, stream, a); \
  } while (0)
  if (a.D == 128) {
    if (k_eq_v) GA_ROWS16_LAUNCH(128, true); else GA_ROWS16_LAUNCH(128, false);
  } else if (a.D == 256) {
    if (k_eq_v) GA_ROWS16_LAUNCH(256, true); else GA_ROWS16_LAUNCH(256, false);
  } else if (a.D == 512 && k_eq_v) {
    GA_ROWS16_LAUNCH(512, true);
  } else {
    return hipErrorInvalidValue;
  }
#undef GA_ROWS16_LAUNCH
  return hipGetLastError();
}

}  // namespace ga
