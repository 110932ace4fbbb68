// decode_valu.hip -- split-KV flash-decode on the vector ALUs (gfx950, wave64).
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
#include <type_traits>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr float kRescaleLog2 = 8.0f;

constexpr int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Waves per work-group: the default keeps the end-of-split LDS merge buffer at 32 KiB;
// the wide variant doubles it when that still fits in 64 KiB, for launches with few
// work-groups (one split per row) that need more waves in flight per CU.
template <int D, int G>
constexpr int valu_nw_base() { return clampi(8192 / (G * D), 1, 4); }
// The wide variant doubles the waves of small work-groups; only where a lane's
// accumulators stay at 64 (the lanes per key are not clamped at D / 8), else it spills.
template <int D, int G>
constexpr bool valu_nw_wide_ok() {
  return valu_nw_base<D, G>() == 4 && G * D <= 2048 && G * D / clampi(G * D / 64, 8, D / 8) <= 64;
}

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
template <int D, int G, int NW_, bool KV_SHARED, bool MULTI>
__global__ void __launch_bounds__(NW_ * 64)
    decode_valu_kernel(DecodeArgs a) {
  using C = ValuCfg<D, G, NW_>;
  constexpr int L = C::L, DPL = C::DPL, NCH = C::NCH, GPW = C::GPW, NW = C::NW, NG = C::NG;
  constexpr int ROW16 = D / 8;  // 16-byte chunks per cache row

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];

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
  AppendRow app;
  app.load(a, b, g, new_slot, threadIdx.x, split == 0);
  const RowRange r = unit_range(a, b, chunk);
  const int k_begin = split * a.split_keys;
  const int k_end = min(r.n, k_begin + a.split_keys);
  if (k_begin >= k_end) {
    if (S == 1) {  // the only split of an empty unit: the output is 0
      for (int idx = threadIdx.x; idx < G * D; idx += NW * 64)
        if (row_active(idx / D)) a.out[row_index(idx / D) * D + idx % D] = 0.0f;
    }
    app.store(a);
    return;  // with S > 1 the merge never reads splits past the unit's end
  }
  __shared__ int s_next;  // next wave-step to hand out
  if (threadIdx.x == 0) s_next = 0;
  __syncthreads();

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

  // Query heads of this KV head, as packed bf16 pairs, in this lane's element order.
  uint32_t qr[G][DPL / 2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + row_index(hh) * D);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint4 v = qp[c * L + j];
      qr[hh][4 * c + 0] = v.x;
      qr[hh][4 * c + 1] = v.y;
      qr[hh][4 * c + 2] = v.z;
      qr[hh][4 * c + 3] = v.w;
    }
  }

  const size_t row0 = (size_t)(b * a.Hkv + g) * a.cap;
  const uint4* kbase = reinterpret_cast<const uint4*>(a.k) + row0 * ROW16;
  const uint4* vbase = reinterpret_cast<const uint4*>(KV_SHARED ? a.k : a.v) + row0 * ROW16;
  // fused append: the appended token's rows, read in place of its slot
  const size_t unit = (size_t)b * a.Hkv + g;
  const uint4* knew = a.new_pos ? reinterpret_cast<const uint4*>(a.k_new) + unit * ROW16 : kbase;
  const uint4* vnew =
      a.new_pos ? reinterpret_cast<const uint4*>(KV_SHARED ? a.k_new : a.v_new) + unit * ROW16
                : vbase;

  float acc[G][DPL];
  float m[G], l[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;
  }

  // Wave-step s covers keys k_begin + s * GPW + grp (one per lane group).  Steps are
  // handed out to waves as they ask for them (an LDS counter), so waves that the SIMD
  // arbiter serves less still finish together with the others; in deterministic mode the
  // order is static (wave w takes w, w + NW, ...), which fixes the summation order.
  const int n_wsteps = (k_end - k_begin + GPW - 1) / GPW;
  const float scale = a.scale;
  const float softcap = a.softcap, inv_softcap = a.inv_softcap;
  int taken = 0;
  auto grab = [&]() -> int {
    if (a.deterministic) return wave + NW * (taken++);
    int s = 0;
    if (lane == 0) s = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(s);
  };

  auto load = [&](uint4(&kr)[NCH], uint4(&vr)[NCH], int step) {
    const int i = k_begin + step * GPW + grp;
    const int ic = i < k_end ? i : k_end - 1;  // past the end: re-read a valid row
    const int slot = key_slot(r, ic, a.cap);
    const bool fresh = slot == new_slot;
    const uint4* kp = fresh ? knew : kbase + (size_t)slot * ROW16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) kr[c] = kp[c * L + j];
    if constexpr (!KV_SHARED) {
      const uint4* vp = fresh ? vnew : vbase + (size_t)slot * ROW16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) vr[c] = vp[c * L + j];
    }
  };

  auto compute = [&](const uint4(&kr)[NCH], const uint4(&vr)[NCH], int step) {
    const int i = k_begin + step * GPW + grp;
    const bool valid = i < k_end;
    const int pos = r.lo + i;  // absolute position of the key (MULTI masks)
    float s[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        d0 = dot2_bf16(qr[hh][4 * c + 0], kr[c].x, d0);
        d1 = dot2_bf16(qr[hh][4 * c + 1], kr[c].y, d1);
        d0 = dot2_bf16(qr[hh][4 * c + 2], kr[c].z, d0);
        d1 = dot2_bf16(qr[hh][4 * c + 3], kr[c].w, d1);
      }
      s[hh] = group_sum<L>(d0 + d1);
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
    const uint4(&vv)[NCH] = KV_SHARED ? kr : vr;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t w[4] = {vv[c].x, vv[c].y, vv[c].z, vv[c].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = bf16_lo(w[t]), hi = bf16_hi(w[t]);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          acc[hh][8 * c + 2 * t] = fmaf(p[hh], lo, acc[hh][8 * c + 2 * t]);
          acc[hh][8 * c + 2 * t + 1] = fmaf(p[hh], hi, acc[hh][8 * c + 2 * t + 1]);
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
  uint4 ka[NCH], va[NCH], kb[NCH], vb[NCH];
  int sa = grab();
  load(ka, va, sa);
  int sb = grab();
  while (sb < n_wsteps) {
    load(kb, vb, sb);
    compute(ka, va, sa);
    sa = grab();
    load(ka, va, sa);
    compute(kb, vb, sb);
    sb = grab();
  }
  if (sa < n_wsteps) compute(ka, va, sa);
  app.store(a);

  // Merge the groups of this wave (lanes j, j + L, j + 2L, ... hold the same elements),
  // exchanging values with DPP / permlane swaps on the VALU.
  auto merge_groups = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mo = xor_lane<OFF>(m[hh], lane);
      const float lo = xor_lane<OFF>(l[hh], lane);
      const float mn = fmaxf(m[hh], mo);
      const float fs = m[hh] == -INFINITY ? 0.0f : exp2_fast(m[hh] - mn);
      const float fo = mo == -INFINITY ? 0.0f : exp2_fast(mo - mn);
      l[hh] = l[hh] * fs + lo * fo;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float ao = xor_lane<OFF>(acc[hh][e], lane);
        acc[hh][e] = acc[hh][e] * fs + ao * fo;
      }
      m[hh] = mn;
    }
  };
  if constexpr (L <= 8) merge_groups(std::integral_constant<int, 8>());
  if constexpr (L <= 16) merge_groups(std::integral_constant<int, 16>());
  if constexpr (L <= 32) merge_groups(std::integral_constant<int, 32>());

  // Merge the waves through LDS, then write the output or this split's partial.
  if (lane < L) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float4* dst = reinterpret_cast<float4*>(&s_acc[wave][hh][8 * (c * L + j)]);
        dst[0] = make_float4(acc[hh][8 * c + 0], acc[hh][8 * c + 1], acc[hh][8 * c + 2],
                             acc[hh][8 * c + 3]);
        dst[1] = make_float4(acc[hh][8 * c + 4], acc[hh][8 * c + 5], acc[hh][8 * c + 6],
                             acc[hh][8 * c + 7]);
      }
      if (j == 0) {
        s_m[wave][hh] = m[hh];
        s_l[wave][hh] = l[hh];
      }
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
  if (a.T > 1) {
    if (k_eq_v)
      hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, false, true>), grid, block, 0, stream, a);
  } else {
    if (k_eq_v)
      hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_valu_kernel<D, G, NW, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  constexpr int base = valu_nw_base<D, G>();
  if constexpr (valu_nw_wide_ok<D, G>()) {
    if (a.n_waves == 2 * base) return launch_dgw<D, G, 2 * base>(a, k_eq_v, stream);
  }
  return launch_dgw<D, G, base>(a, k_eq_v, stream);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  switch (a.Gh * a.Tc) {  // query rows per unit
    case 1: return launch_dg<D, 1>(a, k_eq_v, stream);
    case 2: return launch_dg<D, 2>(a, k_eq_v, stream);
    case 4: return launch_dg<D, 4>(a, k_eq_v, stream);
    case 8: return launch_dg<D, 8>(a, k_eq_v, stream);
    case 16: return launch_dg<D, 16>(a, k_eq_v, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
int wide_waves_d(int G) {
  switch (G) {
    case 1: return valu_nw_wide_ok<D, 1>() ? 2 * valu_nw_base<D, 1>() : 0;
    case 2: return valu_nw_wide_ok<D, 2>() ? 2 * valu_nw_base<D, 2>() : 0;
    case 4: return valu_nw_wide_ok<D, 4>() ? 2 * valu_nw_base<D, 4>() : 0;
    case 8: return valu_nw_wide_ok<D, 8>() ? 2 * valu_nw_base<D, 8>() : 0;
    case 16: return valu_nw_wide_ok<D, 16>() ? 2 * valu_nw_base<D, 16>() : 0;
    default: return 0;
  }
}

}  // namespace

bool decode_valu_supported(int D, int G) {
  return (D == 128 || D == 256 || D == 512) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

int decode_valu_wide_waves(int D, int G) {
  switch (D) {
    case 128: return wide_waves_d<128>(G);
    case 256: return wide_waves_d<256>(G);
    case 512: return wide_waves_d<512>(G);
    default: return 0;
  }
}

hipError_t decode_valu_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  if (a.D == 128) return launch_d<128>(a, k_eq_v, stream);
  if (a.D == 256) return launch_d<256>(a, k_eq_v, stream);
  if (a.D == 512) return launch_d<512>(a, k_eq_v, stream);
  return hipErrorInvalidValue;
}

}  // namespace ga
