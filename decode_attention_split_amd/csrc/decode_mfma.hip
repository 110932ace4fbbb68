// decode_mfma.hip -- matrix-core split-KV decode for the K = V global geometry
// (head_dim 512, 16 query heads per KV head, one cached tensor used as keys and values).
//
// Why matrix cores here: 16 query heads share every key, so a key row of 1 KiB feeds
// 2 * 16 * 512 * 2 = 32 KFLOP (q.k and p.v): 32 flop/byte, above the fp32 vector ridge
// of MI355X (~157 TFLOP/s over 8 TB/s ~ 20 flop/byte), so a VALU kernel cannot reach
// the HBM roofline ("Gemma4-26B-A4B on Apple Silicon", Results, Break 4: 16 query heads
// on one shared K/V head, no separate value projection).
//
// Work partition: the valid keys of all (batch row, KV head) units are laid end to end
// (prefix sums of the per-unit counts, computed on the device from ctx_lens / q_pos) and
// cut into gridDim.x equal chunks, one per work-group.  Ragged contexts with few units
// (a single KV head, batch 16-32) therefore still spread evenly over every CU -- the
// failure mode of decode kernels that ignore key splitting ("Gemma 4 12B (unified
// multimodal)" record, item (4): 2 of 132 SMs busy).  A unit cut across work-groups is
// finished by merge_units_kernel (log-sum-exp); a unit inside one work-group is written
// directly.  Partial slot of (work-group i, unit u) is i + u: slots never collide.
//
// Per wave, 16-key tiles:
//   S^T[16 keys][16 heads] = K[16][512] . Q^T[512][16] with v_mfma_f32_16x16x32_bf16:
//     lane l loads key (l % 16), d = 32 j + 8 (l / 16) + 0..7 for j < 16 straight into the
//     A operand (16-byte loads), Q^T is held in registers in the same d order;
//   the same registers are written once to LDS (row stride 1056 B);
//   O^T[512][16] += V^T[512][16 keys] . P^T[16 keys][16 heads] with
//     v_mfma_f32_16x16x16_bf16: the A operand comes from LDS with ds_read_b64_tr_b16
//     (lanes 4e..4e+3 of a 16-lane block read 16 consecutive d of key e; lane i then holds
//     the 4 keys at column d0 + i), and the B operand is P exactly as the S^T MFMA left it
//     (lane l: head l % 16, keys 4 (l / 16) + 0..3).  P is split into bf16 hi + lo parts
//     so the probabilities keep ~16 mantissa bits; the bf16 cache data is exact.
// The K = V row is read from HBM once and used for both products.  Softmax state per
// head is fp32 in log2 units with lazy rescaling (max raised only past +8).
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int MD = 512;        // head_dim
constexpr int MG = 16;         // query heads per KV head
constexpr int TK = 16;         // keys per tile
constexpr int MNW = 4;         // waves per work-group
constexpr int ROWB = 1056;     // LDS bytes per tile row: 1024 + 32 (bank spread of tr reads)
constexpr int TILE_LDS = TK * ROWB;
constexpr float kRescaleLog2 = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // RNE
}

__device__ __forceinline__ floatx4_t mfma_k32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma_k16(short4_t a, short4_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Valid-key count of unit u (batch row b = u / Hkv).
__device__ __forceinline__ int unit_keys(const DecodeArgs& a, int u) {
  const int b = u / a.Hkv;
  return row_range(a.ctx[b], a.q_pos[b], a.window, a.kind, a.cap, a.max_keys).n;
}

__device__ __forceinline__ int chunk_keys(int T, int NB) {
  const int per = (T + NB - 1) / NB;
  return T > 0 ? (per + TK - 1) / TK * TK : TK;
}

__global__ void __launch_bounds__(MNW * 64, 1) decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char s_tiles[MNW * TILE_LDS];
  __shared__ int s_pref[kMfmaMaxUnits + 1];
  __shared__ float s_m[MNW][MG];
  __shared__ float s_l[MNW][MG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.B * a.Hkv;

  // ---- prefix sums of valid keys per unit (every work-group computes them)
  for (int u = tid; u < R; u += MNW * 64) s_pref[u + 1] = unit_keys(a, u);
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 1; base <= R; base += 64) {
      const int idx = base + lane;
      int v = idx <= R ? s_pref[idx] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
      }
      if (idx <= R) s_pref[idx] = v + carry;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
  const int T = s_pref[R];
  if (blockIdx.x == 0)
    for (int u = tid; u <= R; u += MNW * 64) a.plan[u] = s_pref[u];
  const int C = chunk_keys(T, gridDim.x);
  const int a0 = blockIdx.x * C;
  if (a0 >= T) return;
  const int e0 = min(a0 + C, T);

  // first unit whose keys reach past a0
  int lo_u = 0, hi_u = R - 1;
  while (lo_u < hi_u) {
    const int mid = (lo_u + hi_u) >> 1;
    if (s_pref[mid + 1] > a0) hi_u = mid; else lo_u = mid + 1;
  }

  char* my_tile = s_tiles + wave * TILE_LDS;
  char* lds_w = my_tile + l16 * ROWB + lg * 16;                    // A-operand row writes
  char* lds_r = my_tile + (4 * lg + (l16 >> 2)) * ROWB + (l16 & 3) * 8;  // transposed reads

  for (int u = lo_u; u < R && s_pref[u] < e0; ++u) {
    const int seg_lo = max(a0, s_pref[u]) - s_pref[u];
    const int seg_hi = min(e0, s_pref[u + 1]) - s_pref[u];
    if (seg_hi <= seg_lo) continue;  // empty unit (uniform across the work-group)
    const int b = u / a.Hkv, g = u % a.Hkv;
    const RowRange r = row_range(a.ctx[b], a.q_pos[b], a.window, a.kind, a.cap, a.max_keys);
    const size_t head0 = (size_t)b * a.Hq + (size_t)g * MG;

    // Q^T operand: head l16, d = 32 j + 8 lg + 0..7
    uint4 qv[16];
    {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + (head0 + l16) * MD);
#pragma unroll
      for (int j = 0; j < 16; ++j) qv[j] = qp[4 * j + lg];
    }
    const uint4* kbase = reinterpret_cast<const uint4*>(a.k) + (size_t)u * a.cap * (MD / 8);

    floatx4_t acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    const int n_tiles = (seg_hi - seg_lo + TK - 1) / TK;
    const int nt = n_tiles > wave ? (n_tiles - wave + MNW - 1) / MNW : 0;  // this wave's tiles

    auto load = [&](uint4(&rg)[16], int t) {
      const int key = seg_lo + (wave + MNW * t) * TK + l16;
      const int kc = key < seg_hi ? key : seg_hi - 1;
      const uint4* rp = kbase + (size_t)key_slot(r, kc, a.cap) * (MD / 8);
#pragma unroll
      for (int j = 0; j < 16; ++j) rg[j] = rp[4 * j + lg];
    };

    auto process = [&](uint4(&rg)[16], int t) {
      const int k0 = seg_lo + (wave + MNW * t) * TK;
      // logits of 16 keys x 16 heads
      floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 16; ++j) s = mfma_k32(rg[j], qv[j], s);
      // keep the tile in LDS for the transposed P.V reads, then refill the registers
#pragma unroll
      for (int j = 0; j < 16; ++j) *reinterpret_cast<uint4*>(lds_w + j * 64) = rg[j];
      if (t + 2 < nt) load(rg, t + 2);
      // softmax: lane holds head l16, keys k0 + 4 lg + i
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[i] * a.scale;
        if (a.softcap > 0.0f) v = softcap_tanh(v, a.softcap, a.inv_softcap);
        x[i] = (k0 + 4 * lg + i < seg_hi) ? v * kLog2e : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (mx > m + kRescaleLog2) {
        const float f = exp2_fast(m - mx);
        l *= f;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= f;
        m = mx;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2_fast(x[i] - m);
        l += p[i];
      }
      const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
      const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
      const short4_t ph = __builtin_bit_cast(short4_t, make_uint2(h01, h23));
      const short4_t pl = __builtin_bit_cast(short4_t, make_uint2(l01, l23));
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const short4_t va =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(lds_r + db * 32));
        acc[db] = mfma_k16(va, ph, acc[db]);
        acc[db] = mfma_k16(va, pl, acc[db]);
      }
    };

    uint4 ra[16], rb[16];
    if (nt > 0) load(ra, 0);
    if (nt > 1) load(rb, 1);
    for (int t = 0; t < nt; t += 2) {
      process(ra, t);
      if (t + 1 >= nt) break;
      process(rb, t + 1);
    }

    // ---- merge the waves of this work-group for this unit segment
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (lane < MG) {
      s_m[wave][lane] = m;
      s_l[wave][lane] = l;
    }
    __syncthreads();  // also: every wave is done with its tile LDS
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < MNW; ++w) M = fmaxf(M, s_m[w][l16]);
    float Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < MNW; ++w) {
      const float mw = s_m[w][l16];
      Lsum += mw == -INFINITY ? 0.0f : s_l[w][l16] * exp2_fast(mw - M);
    }
    const float fown = m == -INFINITY ? 0.0f : exp2_fast(m - M);
    floatx4_t* buf0 = reinterpret_cast<floatx4_t*>(s_tiles);             // 32 KiB
    floatx4_t* buf1 = reinterpret_cast<floatx4_t*>(s_tiles + 32 * 1024);  // 32 KiB
    if (wave >= 2) {
      floatx4_t* dst = wave == 2 ? buf0 : buf1;
#pragma unroll
      for (int db = 0; db < 32; ++db) dst[db * 64 + lane] = acc[db] * fown;
    }
    __syncthreads();
    if (wave < 2) {
      const floatx4_t* src = wave == 0 ? buf0 : buf1;
#pragma unroll
      for (int db = 0; db < 32; ++db) acc[db] = acc[db] * fown + src[db * 64 + lane];
    }
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int db = 0; db < 32; ++db) buf0[db * 64 + lane] = acc[db];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int db = 0; db < 32; ++db) acc[db] += buf0[db * 64 + lane];
      const bool whole = seg_lo == 0 && seg_hi == r.n;
      if (whole) {
        const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
        float* o = a.out + (head0 + l16) * MD + 4 * lg;
#pragma unroll
        for (int db = 0; db < 32; ++db)
          *reinterpret_cast<floatx4_t*>(o + 16 * db) = acc[db] * inv;
      } else {
        const size_t slot = (size_t)blockIdx.x + u;
        float* o = a.part_acc + (slot * MG + l16) * MD + 4 * lg;
#pragma unroll
        for (int db = 0; db < 32; ++db) *reinterpret_cast<floatx4_t*>(o + 16 * db) = acc[db];
        if (lane < MG) {
          a.part_ml[(slot * MG + lane) * 2 + 0] = M;
          a.part_ml[(slot * MG + lane) * 2 + 1] = Lsum;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next segment's tiles
  }
}

// Finishes the units that were cut across work-groups; writes 0 for empty units.
// One work-group per (unit, head).
__global__ void __launch_bounds__(256) merge_units_kernel(DecodeArgs a) {
  const int u = blockIdx.x / MG, h = blockIdx.x % MG;
  const int R = a.B * a.Hkv;
  const int T = a.plan[R];
  const int P0 = a.plan[u], P1 = a.plan[u + 1];
  const size_t head = ((size_t)(u / a.Hkv) * a.Hq + (size_t)(u % a.Hkv) * MG + h);
  float* out = a.out + head * MD;
  if (P1 <= P0) {
    for (int d = threadIdx.x; d < MD; d += 256) out[d] = 0.0f;
    return;
  }
  const int C = chunk_keys(T, a.n_blocks);
  const int i0 = P0 / C, i1 = (P1 - 1) / C;
  if (i0 == i1) return;  // written directly by the decode kernel
  float M = -INFINITY;
  for (int i = i0; i <= i1; ++i) M = fmaxf(M, a.part_ml[(((size_t)i + u) * MG + h) * 2]);
  float L = 0.0f;
  for (int i = i0; i <= i1; ++i) {
    const size_t sl = ((size_t)i + u) * MG + h;
    L += a.part_ml[sl * 2 + 1] * exp2_fast(a.part_ml[sl * 2] - M);
  }
  const float inv = 1.0f / L;
  for (int d = threadIdx.x; d < MD; d += 256) {
    float o = 0.0f;
    for (int i = i0; i <= i1; ++i) {
      const size_t sl = ((size_t)i + u) * MG + h;
      o = fmaf(exp2_fast(a.part_ml[sl * 2] - M), a.part_acc[sl * MD + d], o);
    }
    out[d] = o * inv;
  }
}

}  // namespace

bool decode_mfma_supported(int D, int G, bool k_eq_v) { return D == MD && G == MG && k_eq_v; }

size_t decode_mfma_workspace_bytes(int B, int Hkv) {
  const size_t units = (size_t)B * Hkv;
  const size_t slots = (size_t)kMfmaBlocks + units;
  return slots * MG * MD * 4 + slots * MG * 2 * 4 + (units + 1) * 4;
}

hipError_t decode_mfma_launch(const DecodeArgs& a0, hipStream_t stream) {
  DecodeArgs a = a0;
  const long long R = (long long)a.B * a.Hkv;
  if (R <= 0) return hipSuccess;
  if (R > kMfmaMaxUnits) return hipErrorInvalidValue;
  a.n_blocks = kMfmaBlocks;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(kMfmaBlocks), dim3(MNW * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_units_kernel, dim3((unsigned)(R * MG)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ga
