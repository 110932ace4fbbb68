// api.hip -- the C ABI of libgemma_attn: argument checks, split planning and launches.
// Every check that needs no device runs first, so a bad call is rejected before any
// HIP call is made; nothing is launched on error.  The library never allocates, frees
// or synchronises; all work is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "ga_internal.h"
#include "gemma_attn.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device result of the architecture check: 0 unknown, 1 gfx950, -1 other; and the
// device's compute-unit count (read with it).
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

// Work-groups wanted to cover the chip: one per CU.  Plans made before the device is
// known (workspace sizes, host-side checks) assume the most CUs a gfx950 device has, so
// the workspace they size covers any launch on a device with fewer.
constexpr int kTargetBlocks = ga::kMaxBlocks;
constexpr int kMaxSplitKeys = 65536;
#ifndef GA_MULTI_MAX_ROWS
#define GA_MULTI_MAX_ROWS 8
#endif
constexpr int kMultiMaxRows = GA_MULTI_MAX_ROWS;  // multi-token: query rows per unit
constexpr int kMaxTokens = 4096;  // multi-token: query tokens per row

int32_t check_arch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return GA_ERR_ARCH;
  }
  if (dev >= kMaxDevices) return GA_ERR_ARCH;
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return GA_ERR_ARCH;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    const int cus = prop.multiProcessorCount;
    g_cus[dev].store(cus < 1 ? 1 : (cus > ga::kMaxBlocks ? ga::kMaxBlocks : cus),
                     std::memory_order_relaxed);
    g_arch_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? GA_OK : GA_ERR_ARCH;
}

// Compute units of the current device (after a successful check_arch), at most kMaxBlocks.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kTargetBlocks;
  const int c = g_cus[dev].load(std::memory_order_relaxed);
  return c > 0 ? c : kTargetBlocks;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// head sizes 128 (test matrix of the "Gemma support" pull request), 256 (sliding layers)
// and 512 (global layers)
bool head_dim_ok(int d) { return d == 128 || d == 256 || d == 512; }

int32_t check_shape(const ga_shape* s, int32_t window, int32_t T = 1) {
  if (!s) return GA_ERR_NULL;
  if (s->batch < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->capacity <= 0)
    return GA_ERR_DIMS;
  if (!head_dim_ok(s->head_dim)) return GA_ERR_HEAD_DIM;
  if (s->num_q_heads % s->num_kv_heads != 0) return GA_ERR_GQA;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (!ga::decode_valu_supported(s->head_dim, G)) return GA_ERR_GQA;
  if (s->kind != GA_CACHE_LINEAR && s->kind != GA_CACHE_RING) return GA_ERR_KIND;
  if (s->max_ctx < 0) return GA_ERR_MAX_CTX;
  const long long max_ctx = s->max_ctx == 0 ? s->capacity : s->max_ctx;
  if (s->kind == GA_CACHE_LINEAR && max_ctx > s->capacity) return GA_ERR_MAX_CTX;
  if (T < 1) return GA_ERR_DIMS;
  if (T > kMaxTokens) return GA_ERR_TOO_LARGE;
  if (s->kind == GA_CACHE_RING) {
    if (window > s->capacity) return GA_ERR_WINDOW;
    if (window <= 0 && max_ctx > s->capacity) return GA_ERR_WINDOW;
    // T tokens at ctx - T .. ctx - 1: the first one's window starts T - 1 positions before
    // the last one's, so a ring that the context can overrun must keep w + T - 1 slots
    if (window > 0 && max_ctx > s->capacity && (long long)window + T - 1 > s->capacity)
      return GA_ERR_WINDOW;
  }
  // 32-bit index and grid limits
  const long long rows = (long long)s->batch * s->num_kv_heads * s->capacity;
  if (rows * s->head_dim / 8 > (1LL << 40) ||
      (long long)s->batch * T * s->num_q_heads > (1LL << 30))
    return GA_ERR_TOO_LARGE;
  return GA_OK;
}

struct Plan {
  int impl;        // GA_IMPL_VALU / GA_IMPL_MFMA
  int split_keys;  // Ts
  int n_split;     // S
  int max_keys;    // S * Ts
  int T = 1;       // query tokens per row
  int Tc = 1;      // tokens per unit (multi-token)
  int n_chunks = 1;
  bool rows16 = false;  // multi-token on the matrix cores (16 query rows per unit)
  int mfma_rows = 0;    // global matrix-core path: batch rows per launch
  size_t ws_bytes;
};

// Upper bound on valid keys per row from host-known values only.
long long max_keys_bound(const ga_shape* s, int32_t window) {
  long long n = s->max_ctx == 0 ? s->capacity : s->max_ctx;
  if (n > s->capacity) n = s->capacity;  // ring: at most W present; linear: at most C
  if (window > 0 && n > window) n = window;
  return n;
}

bool mfma_eligible(const ga_shape* s, bool k_eq_v) {
  const int G = s->num_q_heads / s->num_kv_heads;
  return ga::decode_mfma_supported(s->head_dim, G, k_eq_v) &&
         s->num_kv_heads <= ga::kMfmaMaxUnits;
}

// Tokens per unit for T query tokens: the largest power of two that keeps heads x tokens
// within kMultiMaxRows (one token when the heads alone reach it) and does not exceed the
// power of two at or above T.
int tokens_per_unit(int G, int T) {
  if (T <= 1) return 1;
  int tc = 1;
  while (tc < T && G * tc * 2 <= kMultiMaxRows) tc *= 2;
  return tc;
}

int32_t valu_plan(const ga_shape* s, int32_t window, int ts, int T, Plan* p,
                  int n_blocks = kTargetBlocks) {
  const int G = s->num_q_heads / s->num_kv_heads;
  const int Tc = tokens_per_unit(G, T);
  const int n_chunks = (T + Tc - 1) / Tc;
  long long nmax = max_keys_bound(s, window);
  if (T > 1 && window > 0) {
    // a unit's keys: the union of Tc consecutive tokens' windows
    long long u = max_keys_bound(s, 0);
    if (u > (long long)window + Tc - 1) u = (long long)window + Tc - 1;
    nmax = u;
  }
  const long long units = (long long)s->batch * s->num_kv_heads * n_chunks;
  if (ts == 0) {
    // Enough work-groups to reach every CU (whole 64-key splits: the per-split partial,
    // G * (D + 2) floats, stays small next to the split's KV bytes).  Rows that fit one
    // split are written directly, with no partials and no merge launch.  A small batch is
    // latency-bound: each wave's steps wait on their loads in turn, so shorter splits
    // finish sooner (Gemma-3-1B sliding layer, B 32: 12.0 us at 128 keys, 8.8 at 64).
    long long want_splits = units > 0 ? (n_blocks + units - 1) / units : 1;
    long long t = nmax > 0 ? (nmax + want_splits - 1) / want_splits : 64;
    t = (t + 63) / 64 * 64;
    if (t < 64) t = 64;
    if (t > kMaxSplitKeys) t = kMaxSplitKeys;
    ts = (int)t;
  }
  long long S = nmax > 0 ? (nmax + ts - 1) / ts : 1;
  if (S < 1) S = 1;
  if (S * ts > (1LL << 30) || units * S > (1LL << 31) - 1) return GA_ERR_TOO_LARGE;
  p->impl = GA_IMPL_VALU;
  p->split_keys = ts;
  p->n_split = (int)S;
  p->max_keys = (int)(S * ts);
  p->T = T;
  p->Tc = Tc;
  p->n_chunks = n_chunks;
  p->ws_bytes = S > 1 ? (size_t)s->batch * T * s->num_q_heads * (size_t)S *
                            (size_t)(s->head_dim + 2) * 4u
                      : 0;
  return GA_OK;
}

constexpr int kRows16WavesPerCU = 8;  // waves wanted per CU

// Several tokens on the matrix cores: 16 query rows per unit (16 / G tokens of G heads),
// splits sized so that about kRows16Waves waves cover the chip (each split is one
// work-group of ga::decode_rows16_waves waves).
int32_t rows16_plan(const ga_shape* s, int32_t window, int ts, int T, Plan* p,
                    int n_blocks = kTargetBlocks) {
  const int G = s->num_q_heads / s->num_kv_heads;
  const int Tc = 16 / G;
  const int n_chunks = (T + Tc - 1) / Tc;
  long long nmax = max_keys_bound(s, 0);
  if (window > 0 && nmax > (long long)window + Tc - 1) nmax = (long long)window + Tc - 1;
  const long long units = (long long)s->batch * s->num_kv_heads * n_chunks;
  if (ts == 0) {
    const long long groups =
        (long long)kRows16WavesPerCU * n_blocks / ga::decode_rows16_waves(s->head_dim);
    const long long want = units > 0 ? (groups + units - 1) / units : 1;
    // whole 16-key tiles (the kernel's step), so the last split of a unit is not much
    // shorter than the others; at least 64 keys, so a split outweighs its prologue
    long long t = nmax > 0 ? (nmax + want - 1) / want : 64;
    t = (t + 15) / 16 * 16;
    if (t < 64) t = 64;
    if (t > kMaxSplitKeys) t = kMaxSplitKeys;
    ts = (int)t;
  }
  long long S = nmax > 0 ? (nmax + ts - 1) / ts : 1;
  if (S < 1) S = 1;
  if (S * ts > (1LL << 30) || units * S > (1LL << 31) - 1) return GA_ERR_TOO_LARGE;
  p->impl = GA_IMPL_MFMA;
  p->rows16 = true;
  p->split_keys = ts;
  p->n_split = (int)S;
  p->max_keys = (int)(S * ts);
  p->T = T;
  p->Tc = Tc;
  p->n_chunks = n_chunks;
  p->ws_bytes = S > 1 ? (size_t)s->batch * T * s->num_q_heads * (size_t)S *
                            (size_t)(s->head_dim + 2) * 4u
                      : 0;
  return GA_OK;
}

// Global K = V geometry on the matrix cores: balanced over the chip (ts = 0) or in
// splits of ts keys.  One launch covers at most ga::kMfmaMaxUnits units (whole rows), and
// at most 2^31 - 1 keys in all; larger batches run as several launches that reuse the
// workspace, which is sized for one.
int32_t mfma_plan(const ga_shape* s, int32_t window, int ts, int n_blocks, Plan* p) {
  long long nmax = max_keys_bound(s, window);
  if (nmax < 1) nmax = 1;
  long long rows = ga::kMfmaMaxUnits / s->num_kv_heads;
  const long long by_keys = ((1LL << 31) - 1) / (nmax * s->num_kv_heads);
  if (rows > by_keys) rows = by_keys;
  if (rows < 1) return GA_ERR_TOO_LARGE;
  if (rows > s->batch) rows = s->batch;
  const long long units = rows * s->num_kv_heads;
  const long long grid = ga::decode_mfma_grid((int)units, n_blocks, ts, (int)nmax);
  if (grid > (1LL << 31) - 1) return GA_ERR_TOO_LARGE;
  p->impl = GA_IMPL_MFMA;
  p->split_keys = ts;
  p->n_split = 0;
  p->max_keys = (int)nmax;
  p->mfma_rows = (int)rows;
  p->ws_bytes = units > 0 ? ga::decode_mfma_workspace_bytes(grid, (int)units) : 0;
  return GA_OK;
}

// k_eq_v: 1 / 0 when known (a decode call), -1 for a workspace query, which then sizes
// for whichever implementation AUTO may pick.
int32_t make_plan(const ga_shape* s, int32_t window, const ga_decode_opts* o, int k_eq_v,
                  Plan* p, int T = 1, int n_blocks = kTargetBlocks) {
  int impl = GA_IMPL_AUTO, ts = 0;
  if (o) {
    for (int i = 0; i < 5; ++i)
      if (o->reserved[i] != 0) return GA_ERR_OPTS;
    if (o->deterministic != 0 && o->deterministic != 1) return GA_ERR_OPTS;
    impl = o->impl;
    ts = o->split_keys;
    if (impl < GA_IMPL_AUTO || impl > GA_IMPL_MFMA) return GA_ERR_OPTS;
    if (ts != 0 && (ts < 64 || ts > kMaxSplitKeys || ts % 64 != 0)) return GA_ERR_OPTS;
  }
  if (T > 1) {
    // several query tokens (per-row masks): 16 query rows per unit on the matrix cores
    // when heads x tokens fill at least a quarter of them (measured on the 12B sliding
    // layer with 2 and 4 heads per KV head: the matrix cores win from 4 rows on, by up
    // to 4x), else the vector kernel
    const int G = s->num_q_heads / s->num_kv_heads;
    const bool ok = k_eq_v != -1 ? ga::decode_rows16_supported(s->head_dim, k_eq_v == 1)
                                 : ga::decode_rows16_supported(s->head_dim, false) ||
                                       ga::decode_rows16_supported(s->head_dim, true);
    if (impl == GA_IMPL_MFMA) {
      if (!ok) return GA_ERR_OPTS;
      return rows16_plan(s, window, ts, T, p, n_blocks);
    }
    if (impl == GA_IMPL_AUTO && ok && (long long)G * T >= 4) {
      if (k_eq_v != -1) return rows16_plan(s, window, ts, T, p, n_blocks);
      Plan v;  // workspace query: size for whichever the call may pick
      int32_t st = valu_plan(s, window, ts, T, &v, n_blocks);
      if (st != GA_OK) return st;
      st = rows16_plan(s, window, ts, T, p, n_blocks);
      if (st != GA_OK) return st;
      if (v.ws_bytes > p->ws_bytes) p->ws_bytes = v.ws_bytes;
      return GA_OK;
    }
    return valu_plan(s, window, ts, T, p, n_blocks);
  }
  if (impl == GA_IMPL_MFMA) {
    // the matrix-core kernel balances keys over the chip, or takes the given split size
    if (k_eq_v == 0 || !mfma_eligible(s, true)) return GA_ERR_OPTS;
    return mfma_plan(s, window, ts, n_blocks, p);
  }
  if (impl == GA_IMPL_AUTO && k_eq_v != 0 && mfma_eligible(s, true)) {
    // the global K = V geometry stays on the matrix cores for every batch and split size
    if (k_eq_v == 1) return mfma_plan(s, window, ts, n_blocks, p);
    Plan v;  // workspace query: K = V is not known yet, size for either kernel
    int32_t st = valu_plan(s, window, ts, 1, &v, n_blocks);
    if (st != GA_OK) return st;
    st = mfma_plan(s, window, ts, n_blocks, p);
    if (st != GA_OK) return st;
    if (v.ws_bytes > p->ws_bytes) p->ws_bytes = v.ws_bytes;
    return GA_OK;
  }
  return valu_plan(s, window, ts, 1, p, n_blocks);
}

}  // namespace

extern "C" {

int32_t gemma_attn_version(void) { return 200; }

const char* gemma_attn_strerror(int32_t st) {
  switch (st) {
    case GA_OK: return "ok";
    case GA_ERR_NULL: return "a required pointer is NULL or not 16-byte aligned";
    case GA_ERR_DIMS: return "invalid dimensions (batch < 0, or a head count or capacity <= 0)";
    case GA_ERR_HEAD_DIM: return "head_dim must be 128, 256 or 512";
    case GA_ERR_GQA: return "num_q_heads must be num_kv_heads times 1, 2, 4, 8 or 16";
    case GA_ERR_KIND: return "cache kind must be GA_CACHE_LINEAR or GA_CACHE_RING";
    case GA_ERR_WINDOW:
      return "ring cache: window exceeds the ring capacity, full attention while the "
             "context can exceed it, or (several tokens) window + tokens - 1 exceeds it";
    case GA_ERR_WORKSPACE: return "workspace missing or smaller than ga_decode_workspace_bytes";
    case GA_ERR_SCALE: return "scale must be finite";
    case GA_ERR_V_MISMATCH: return "v_cache and v_new must both be NULL (K = V) or both set";
    case GA_ERR_ARCH: return "no HIP device, or the current device is not gfx950 (MI355X)";
    case GA_ERR_LAUNCH: return "kernel launch failed";
    case GA_ERR_OPTS: return "decode options invalid or unsupported for this shape";
    case GA_ERR_MAX_CTX: return "max_ctx must be >= 0 and, for a linear cache, <= capacity";
    case GA_ERR_TOO_LARGE: return "sizes overflow the kernels' index or grid range";
    case GA_ERR_SCRATCH:
      return "the call needs more workspace than the fixed device scratch of "
             "gemma_attn_decode_noalloc holds (GA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t ga_decode_workspace_bytes(const ga_shape* shape, int32_t window,
                                 const ga_decode_opts* opts) {
  if (check_shape(shape, window) != GA_OK) return SIZE_MAX;
  Plan p;
  if (make_plan(shape, window, opts, -1, &p) != GA_OK) return SIZE_MAX;
  return p.ws_bytes;
}

size_t ga_decode_multi_workspace_bytes(const ga_shape* shape, int32_t num_tokens, int32_t window,
                                       const ga_decode_opts* opts) {
  if (check_shape(shape, window, num_tokens) != GA_OK) return SIZE_MAX;
  Plan p;
  if (make_plan(shape, window, opts, -1, &p, num_tokens) != GA_OK) return SIZE_MAX;
  return p.ws_bytes;
}

size_t ga_decode_fp8_workspace_bytes(const ga_shape* shape, int32_t num_tokens, int32_t window,
                                     const ga_decode_opts* opts) {
  if (check_shape(shape, window, num_tokens) != GA_OK) return SIZE_MAX;
  Plan p;
  if (make_plan(shape, window, opts, -1, &p, num_tokens) != GA_OK) return SIZE_MAX;
  return p.ws_bytes;
}

}  // extern "C"

namespace {

// fp8 e4m3 caches: codes and float32 row scales of K, and of V unless K = V.
struct Fp8Cache {
  const uint8_t* k;
  const float* ks;
  const uint8_t* v;
  const float* vs;
};

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Rotary embedding applied to q and the appended K row before the decode (single token,
// bf16 caches): the rotated q goes to q_out.
struct RopeIn {
  ga_bf16* q_out;
  const double* table;  // [B, dim / 2] (cos, sin) pairs at pos[b]
  int dim;
};

// Decode, optionally fused with the cache append of one token per row (k_new != nullptr),
// over bf16 caches (k_cache / v_cache) or fp8 caches (f8 != nullptr).
int32_t decode_impl(const ga_shape* shape, const ga_bf16* q, ga_bf16* k_cache, ga_bf16* v_cache,
                    const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* new_pos,
                    const int32_t* ctx_lens, const int32_t* q_pos, int32_t window, float softcap,
                    float scale, float* out, void* workspace, size_t workspace_bytes,
                    const ga_decode_opts* opts, void* stream, int32_t T = 1,
                    const Fp8Cache* f8 = nullptr, const RopeIn* rope = nullptr) {
  int32_t st = check_shape(shape, window, T);
  if (st != GA_OK) return st;
  if (f8) {
    if (!f8->k || !f8->ks) return GA_ERR_NULL;
    if ((f8->v == nullptr) != (f8->vs == nullptr)) return GA_ERR_V_MISMATCH;
    if (!aligned16(f8->k) || !aligned16(f8->v) || !aligned4(f8->ks) || !aligned4(f8->vs))
      return GA_ERR_NULL;
    // the bf16 cache checks below look at the codes (never dereferenced as bf16)
    k_cache = reinterpret_cast<ga_bf16*>(const_cast<uint8_t*>(f8->k));
    v_cache = reinterpret_cast<ga_bf16*>(const_cast<uint8_t*>(f8->v));
  }
  if (!q || !k_cache || !ctx_lens || !q_pos || !out) return GA_ERR_NULL;
  if (k_new) {
    if (!new_pos) return GA_ERR_NULL;
    if ((v_cache == nullptr) != (v_new == nullptr)) return GA_ERR_V_MISMATCH;
    if (!aligned16(k_new) || !aligned16(v_new)) return GA_ERR_NULL;
  }
  if (!aligned16(q) || !aligned16(k_cache) || (v_cache && !aligned16(v_cache)) ||
      !aligned16(out) || !aligned16(workspace))
    return GA_ERR_NULL;
  if (!std::isfinite(scale)) return GA_ERR_SCALE;
  const bool k_eq_v = v_cache == nullptr || v_cache == k_cache;
  Plan p;
  st = make_plan(shape, window, opts, k_eq_v ? 1 : 0, &p, T);
  if (st != GA_OK) return st;
  const int D = shape->head_dim;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return GA_ERR_WORKSPACE;
  st = check_arch();
  if (st != GA_OK) return st;
  if (shape->batch == 0) return GA_OK;
  const int n_blocks = device_cus();
  if (n_blocks != kTargetBlocks) {
    // fewer CUs than the plan assumed: the same choices with fewer work-groups, which
    // need no more workspace than was checked above
    st = make_plan(shape, window, opts, k_eq_v ? 1 : 0, &p, T, n_blocks);
    if (st != GA_OK) return st;
  }

  ga::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = k_eq_v ? k_cache : v_cache;
  a.ctx = ctx_lens;
  a.q_pos = q_pos;
  a.out = out;
  float* ws = static_cast<float*>(workspace);
  a.part_acc = nullptr;
  a.part_ml = nullptr;
  a.plan = nullptr;
  a.n_blocks = 0;
  if (p.impl == GA_IMPL_MFMA && !p.rows16) {
    const size_t slots = (size_t)ga::decode_mfma_grid(p.mfma_rows * shape->num_kv_heads,
                                                      n_blocks, p.split_keys, p.max_keys);
    a.part_acc = ws;
    a.part_ml = ws + slots * 16 * D;
    a.plan = reinterpret_cast<int*>(a.part_ml + slots * 16 * 2);
    a.n_blocks = n_blocks;
    a.launch_rows = p.mfma_rows;
  } else if (p.n_split > 1) {
    const size_t n_acc = (size_t)shape->batch * T * shape->num_q_heads * (size_t)p.n_split * D;
    a.part_acc = ws;
    a.part_ml = ws + n_acc;
  }
  a.B = shape->batch;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.D = D;
  a.cap = shape->capacity;
  a.kind = shape->kind;
  a.window = window;
  a.scale = scale;
  const bool cap_on = std::isfinite(softcap) && softcap > 0.0f;
  a.softcap = cap_on ? softcap : 0.0f;
  a.inv_softcap = cap_on ? 1.0f / softcap : 0.0f;
  a.split_keys = p.split_keys;
  a.n_split = p.n_split;
  a.max_keys = p.max_keys;
  a.deterministic = opts ? opts->deterministic : 0;
  a.T = p.T;
  a.Tc = p.Tc;
  a.n_chunks = p.n_chunks;
  a.Gh = shape->num_q_heads / shape->num_kv_heads;
  a.max_union = p.max_keys;
  if (f8) {
    a.fp8 = 1;
    a.k8 = f8->k;
    a.k_scale = f8->ks;
    a.v8 = k_eq_v ? f8->k : f8->v;
    a.v_scale = k_eq_v ? f8->ks : f8->vs;
  }
  a.k_new = k_new;
  a.v_new = k_eq_v ? nullptr : v_new;
  a.new_pos = k_new ? new_pos : nullptr;
  a.k_dst = k_cache;
  a.v_dst = k_eq_v ? nullptr : v_cache;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (f8 && k_new) {
    // The quantizing append runs inside the single-token launch (vector kernel, or the
    // matrix-core kernel of the global geometry); before the multi-token matrix-core
    // decode it is its own launch.
    if (!p.rows16 && T == 1) {
      a.k8_dst = const_cast<uint8_t*>(f8->k);
      a.ks_dst = const_cast<float*>(f8->ks);
      a.v8_dst = k_eq_v ? nullptr : const_cast<uint8_t*>(f8->v);
      a.vs_dst = k_eq_v ? nullptr : const_cast<float*>(f8->vs);
      a.k_dst = nullptr;  // no bf16 row moves
      a.v_dst = nullptr;
    } else {
      e = ga::append_fp8_launch(a.B, 1, a.Hkv, D, a.cap, a.kind, const_cast<uint8_t*>(f8->k),
                                const_cast<float*>(f8->ks),
                                k_eq_v ? nullptr : const_cast<uint8_t*>(f8->v),
                                k_eq_v ? nullptr : const_cast<float*>(f8->vs), k_new,
                                k_eq_v ? nullptr : v_new, new_pos, s);
      if (e != hipSuccess) return GA_ERR_LAUNCH;
      a.k_new = nullptr;
      a.v_new = nullptr;
      a.new_pos = nullptr;
    }
  }
  if (rope) {
    // Fused into the single-token launch (vector kernel, or the matrix-core kernel on
    // bf16 caches); every work-group of a unit rotates from q, so an in-place q_out needs
    // a single split (the matrix-core kernel has several per unit: never in place).
    // Otherwise the RoPE + append kernel runs first and the decode reads the rotated q
    // and the appended cache.
    const bool separate_out = (const void*)rope->q_out != (const void*)q;
    const bool fused = !p.rows16 && (p.impl == GA_IMPL_MFMA ? !f8 && separate_out
                                                            : p.n_split == 1 || separate_out);
    if (fused) {
      a.rope = 1;
      a.rope_dim = rope->dim;
      a.rope_table = rope->table;
      a.q_rot_out = rope->q_out;
    } else {
      // (the base is not read: with one token every angle comes from the table)
      e = ga::rope_append_launch(a.B, 1, a.Hq, a.Hkv, D, a.cap, a.kind, rope->dim, 1.0, q,
                                 rope->q_out, k_cache, k_eq_v ? nullptr : v_cache, k_new,
                                 k_eq_v ? nullptr : v_new, new_pos, rope->table, s);
      if (e != hipSuccess) return GA_ERR_LAUNCH;
      a.q = rope->q_out;
      a.k_new = nullptr;
      a.v_new = nullptr;
      a.new_pos = nullptr;
    }
  }
  if (p.rows16) {
    e = ga::decode_rows16_launch(a, k_eq_v, s);
    if (e == hipSuccess && p.n_split > 1) e = ga::merge_launch(a, s);
  } else if (p.impl == GA_IMPL_MFMA) {
    e = ga::decode_mfma_launch(a, s);
  } else {
    e = ga::decode_valu_launch(a, k_eq_v, s);
    if (e == hipSuccess && p.n_split > 1) e = ga::merge_launch(a, s);
  }
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t gemma_attn_decode_ex(const ga_shape* shape, const ga_bf16* q, const ga_bf16* k_cache,
                             const ga_bf16* v_cache, const int32_t* ctx_lens, const int32_t* q_pos,
                             int32_t window, float softcap, float scale, float* out, void* workspace,
                             size_t workspace_bytes, const ga_decode_opts* opts, void* stream) {
  // The caches are only read when nothing is appended.
  return decode_impl(shape, q, const_cast<ga_bf16*>(k_cache), const_cast<ga_bf16*>(v_cache),
                     nullptr, nullptr, nullptr, ctx_lens, q_pos, window, softcap, scale, out,
                     workspace, workspace_bytes, opts, stream);
}

int32_t gemma_attn_decode_append(const ga_shape* shape, const ga_bf16* q, ga_bf16* k_cache,
                                 ga_bf16* v_cache, const ga_bf16* k_new, const ga_bf16* v_new,
                                 const int32_t* pos, const int32_t* ctx_lens,
                                 const int32_t* q_pos, int32_t window, float softcap, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 const ga_decode_opts* opts, void* stream) {
  if (!k_new) return GA_ERR_NULL;
  return decode_impl(shape, q, k_cache, v_cache, k_new, v_new, pos, ctx_lens, q_pos, window,
                     softcap, scale, out, workspace, workspace_bytes, opts, stream);
}

int32_t gemma_attn_decode_rope_append(const ga_shape* shape, const ga_bf16* q, ga_bf16* q_out,
                                      ga_bf16* k_cache, ga_bf16* v_cache, const ga_bf16* k_new,
                                      const ga_bf16* v_new, const int32_t* pos,
                                      const int32_t* ctx_lens, const int32_t* q_pos,
                                      int32_t window, float softcap, float scale,
                                      const double* rope_table, int32_t rotary_dim, float* out,
                                      void* workspace, size_t workspace_bytes,
                                      const ga_decode_opts* opts, void* stream) {
  if (!shape) return GA_ERR_NULL;
  if (!k_new || !q_out) return GA_ERR_NULL;
  if (!aligned16(q_out)) return GA_ERR_NULL;
  if (shape->head_dim > 0 && (rotary_dim < 0 || rotary_dim > shape->head_dim ||
                              rotary_dim % 2 != 0))
    return GA_ERR_OPTS;
  if (rotary_dim > 0 && (!rope_table || !aligned16(rope_table))) return GA_ERR_NULL;
  const RopeIn rope{q_out, rope_table, rotary_dim};
  return decode_impl(shape, q, k_cache, v_cache, k_new, v_new, pos, ctx_lens, q_pos, window,
                     softcap, scale, out, workspace, workspace_bytes, opts, stream, 1, nullptr,
                     &rope);
}

int32_t gemma_attn_decode(const ga_shape* shape, const ga_bf16* q, const ga_bf16* k_cache,
                          const ga_bf16* v_cache, const int32_t* ctx_lens, const int32_t* q_pos,
                          int32_t window, float softcap, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return gemma_attn_decode_ex(shape, q, k_cache, v_cache, ctx_lens, q_pos, window, softcap, scale,
                              out, workspace, workspace_bytes, nullptr, stream);
}

int32_t gemma_kv_append(const ga_shape* shape, ga_bf16* k_cache, ga_bf16* v_cache,
                        const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                        void* stream) {
  if (!shape) return GA_ERR_NULL;
  if (shape->batch < 0 || shape->num_kv_heads <= 0 || shape->num_q_heads <= 0 ||
      shape->capacity <= 0)
    return GA_ERR_DIMS;
  if (!head_dim_ok(shape->head_dim)) return GA_ERR_HEAD_DIM;
  if (shape->kind != GA_CACHE_LINEAR && shape->kind != GA_CACHE_RING) return GA_ERR_KIND;
  if (!k_cache || !k_new || !pos) return GA_ERR_NULL;
  if ((v_cache == nullptr) != (v_new == nullptr)) return GA_ERR_V_MISMATCH;
  if (!aligned16(k_cache) || !aligned16(k_new) || !aligned16(v_cache) || !aligned16(v_new))
    return GA_ERR_NULL;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::append_launch(shape->batch, 1, shape->num_kv_heads, shape->head_dim,
                                   shape->capacity, shape->kind, k_cache, v_cache, k_new, v_new,
                                   pos, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_attn_validate(const ga_shape* shape, const int32_t* ctx_lens, const int32_t* q_pos,
                            int32_t window, int32_t* dev_flags, void* stream) {
  int32_t st = check_shape(shape, window);
  if (st != GA_OK) return st;
  if (!ctx_lens || !q_pos || !dev_flags) return GA_ERR_NULL;
  st = check_arch();
  if (st != GA_OK) return st;
  const int max_ctx = shape->max_ctx == 0 ? shape->capacity : shape->max_ctx;
  hipError_t e = ga::validate_launch(shape->batch, 1, shape->capacity, shape->kind, window,
                                     max_ctx, ctx_lens, q_pos, dev_flags,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_attn_decode_multi(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                                const ga_bf16* k_cache, const ga_bf16* v_cache,
                                const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                                float softcap, float scale, float* out, void* workspace,
                                size_t workspace_bytes, const ga_decode_opts* opts,
                                void* stream) {
  return decode_impl(shape, q, const_cast<ga_bf16*>(k_cache), const_cast<ga_bf16*>(v_cache),
                     nullptr, nullptr, nullptr, ctx_lens, q_pos, window, softcap, scale, out,
                     workspace, workspace_bytes, opts, stream, num_tokens);
}

int32_t gemma_kv_append_multi(const ga_shape* shape, int32_t num_tokens, ga_bf16* k_cache,
                              ga_bf16* v_cache, const ga_bf16* k_new, const ga_bf16* v_new,
                              const int32_t* pos, void* stream) {
  if (!shape) return GA_ERR_NULL;
  if (shape->batch < 0 || shape->num_kv_heads <= 0 || shape->num_q_heads <= 0 ||
      shape->capacity <= 0 || num_tokens < 1)
    return GA_ERR_DIMS;
  if (num_tokens > kMaxTokens) return GA_ERR_TOO_LARGE;
  if (!head_dim_ok(shape->head_dim)) return GA_ERR_HEAD_DIM;
  if (shape->kind != GA_CACHE_LINEAR && shape->kind != GA_CACHE_RING) return GA_ERR_KIND;
  if (!k_cache || !k_new || !pos) return GA_ERR_NULL;
  if ((v_cache == nullptr) != (v_new == nullptr)) return GA_ERR_V_MISMATCH;
  if (!aligned16(k_cache) || !aligned16(k_new) || !aligned16(v_cache) || !aligned16(v_new))
    return GA_ERR_NULL;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::append_launch(shape->batch, num_tokens, shape->num_kv_heads,
                                   shape->head_dim, shape->capacity, shape->kind, k_cache,
                                   v_cache, k_new, v_new, pos, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_attn_decode_fp8(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                              const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales,
                              const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                              float softcap, float scale, float* out, void* workspace,
                              size_t workspace_bytes, const ga_decode_opts* opts, void* stream) {
  const Fp8Cache f8{k_codes, k_scales, v_codes, v_scales};
  return decode_impl(shape, q, nullptr, nullptr, nullptr, nullptr, nullptr, ctx_lens, q_pos,
                     window, softcap, scale, out, workspace, workspace_bytes, opts, stream,
                     num_tokens, &f8);
}

int32_t gemma_attn_decode_append_fp8(const ga_shape* shape, const ga_bf16* q, uint8_t* k_codes,
                                     float* k_scales, uint8_t* v_codes, float* v_scales,
                                     const ga_bf16* k_new, const ga_bf16* v_new,
                                     const int32_t* pos, const int32_t* ctx_lens,
                                     const int32_t* q_pos, int32_t window, float softcap,
                                     float scale, float* out, void* workspace,
                                     size_t workspace_bytes, const ga_decode_opts* opts,
                                     void* stream) {
  if (!k_new) return GA_ERR_NULL;
  const Fp8Cache f8{k_codes, k_scales, v_codes, v_scales};
  return decode_impl(shape, q, nullptr, nullptr, k_new, v_new, pos, ctx_lens, q_pos, window,
                     softcap, scale, out, workspace, workspace_bytes, opts, stream, 1, &f8);
}

int32_t gemma_kv_append_fp8(const ga_shape* shape, int32_t num_tokens, uint8_t* k_codes,
                            float* k_scales, uint8_t* v_codes, float* v_scales,
                            const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                            void* stream) {
  if (!shape) return GA_ERR_NULL;
  if (shape->batch < 0 || shape->num_kv_heads <= 0 || shape->num_q_heads <= 0 ||
      shape->capacity <= 0 || num_tokens < 1)
    return GA_ERR_DIMS;
  if (num_tokens > kMaxTokens) return GA_ERR_TOO_LARGE;
  if (!head_dim_ok(shape->head_dim)) return GA_ERR_HEAD_DIM;
  if (shape->kind != GA_CACHE_LINEAR && shape->kind != GA_CACHE_RING) return GA_ERR_KIND;
  if (!k_codes || !k_scales || !k_new || !pos) return GA_ERR_NULL;
  if ((v_codes == nullptr) != (v_new == nullptr) || (v_codes == nullptr) != (v_scales == nullptr))
    return GA_ERR_V_MISMATCH;
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned4(k_scales) || !aligned4(v_scales))
    return GA_ERR_NULL;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::append_fp8_launch(shape->batch, num_tokens, shape->num_kv_heads,
                                       shape->head_dim, shape->capacity, shape->kind, k_codes,
                                       k_scales, v_codes, v_scales, k_new, v_new, pos,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_rope_append(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                          ga_bf16* q_out, ga_bf16* k_cache, ga_bf16* v_cache,
                          const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                          float rope_base, int32_t rotary_dim, void* stream) {
  if (!shape) return GA_ERR_NULL;
  if (shape->batch < 0 || shape->num_kv_heads <= 0 || shape->num_q_heads <= 0 ||
      shape->capacity <= 0 || num_tokens < 1)
    return GA_ERR_DIMS;
  if (num_tokens > kMaxTokens) return GA_ERR_TOO_LARGE;
  if (!head_dim_ok(shape->head_dim)) return GA_ERR_HEAD_DIM;
  if (shape->num_q_heads % shape->num_kv_heads != 0) return GA_ERR_GQA;
  if (shape->kind != GA_CACHE_LINEAR && shape->kind != GA_CACHE_RING) return GA_ERR_KIND;
  if (rotary_dim < 0 || rotary_dim > shape->head_dim || rotary_dim % 2 != 0 ||
      !(rope_base > 0.0f) || !std::isfinite(rope_base))
    return GA_ERR_OPTS;
  if (!q || !q_out || !pos) return GA_ERR_NULL;
  if ((k_cache == nullptr) != (k_new == nullptr)) return GA_ERR_NULL;  // q only: both NULL
  if ((v_cache == nullptr) != (v_new == nullptr)) return GA_ERR_V_MISMATCH;
  if (!k_cache && v_cache) return GA_ERR_V_MISMATCH;
  if ((long long)shape->batch * num_tokens * (shape->num_q_heads + 2LL * shape->num_kv_heads) >
      (1LL << 31) - 1)
    return GA_ERR_TOO_LARGE;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::rope_append_launch(
      shape->batch, num_tokens, shape->num_q_heads, shape->num_kv_heads, shape->head_dim,
      shape->capacity, shape->kind, rotary_dim, (double)rope_base, q, q_out, k_cache, v_cache,
      k_new, v_new, pos, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_rope_table(int32_t batch, const int32_t* pos, float rope_base, int32_t rotary_dim,
                         int32_t head_dim, double* table, void* stream) {
  if (batch < 0 || rotary_dim < 0 || rotary_dim % 2 != 0) return GA_ERR_DIMS;
  if (!head_dim_ok(head_dim)) return GA_ERR_HEAD_DIM;
  if (rotary_dim > head_dim) return GA_ERR_DIMS;
  if (!(rope_base > 0.0f) || !std::isfinite(rope_base)) return GA_ERR_OPTS;
  if (batch == 0 || rotary_dim == 0) return GA_OK;
  if (!pos || !table) return GA_ERR_NULL;
  if (!aligned16(table)) return GA_ERR_NULL;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::rope_table_launch(batch, rotary_dim, head_dim, (double)rope_base, pos,
                                       table, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_attn_validate_multi(const ga_shape* shape, int32_t num_tokens,
                                  const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                                  int32_t* dev_flags, void* stream) {
  int32_t st = check_shape(shape, window, num_tokens);
  if (st != GA_OK) return st;
  if (!ctx_lens || !q_pos || !dev_flags) return GA_ERR_NULL;
  st = check_arch();
  if (st != GA_OK) return st;
  const int max_ctx = shape->max_ctx == 0 ? shape->capacity : shape->max_ctx;
  hipError_t e = ga::validate_launch(shape->batch, num_tokens, shape->capacity, shape->kind,
                                     window, max_ctx, ctx_lens, q_pos, dev_flags,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

int32_t gemma_attn_debug_ranges(const ga_shape* shape, const int32_t* ctx_lens,
                                const int32_t* q_pos, int32_t window, int32_t* dev_out,
                                void* stream) {
  int32_t st = check_shape(shape, window);
  if (st != GA_OK) return st;
  if (!ctx_lens || !q_pos || !dev_out) return GA_ERR_NULL;
  Plan p;
  st = make_plan(shape, window, nullptr, 0, &p);
  if (st != GA_OK) return st;
  st = check_arch();
  if (st != GA_OK) return st;
  hipError_t e = ga::ranges_launch(shape->batch, shape->capacity, shape->kind, window, p.max_keys,
                                   ctx_lens, q_pos, dev_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}

}  // extern "C"

// ---- allocation-free decode: the same as gemma_attn_decode_ex with the library's own
// device scratch instead of a caller workspace.
namespace {

// The scratch: one copy per device (a __device__ array lives in each device's copy of the
// code object), zero-filled when the code object loads, kept until the process ends.  In
// host code `g_scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
__device__ __attribute__((aligned(256))) unsigned char g_scratch[GA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The scratch's device address on the current device (nullptr on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);  // the same address if two race
  return p;
}

}  // namespace

extern "C" int32_t gemma_attn_decode_noalloc(const ga_shape* shape, const ga_bf16* q,
                                             const ga_bf16* k_cache, const ga_bf16* v_cache,
                                             const int32_t* ctx_lens, const int32_t* q_pos,
                                             int32_t window, float softcap, float scale,
                                             float* out, const ga_decode_opts* opts,
                                             void* stream) {
  // the workspace this call needs, from the same plan gemma_attn_decode_ex makes (all its
  // host checks first, so a bad call returns the same error with nothing launched)
  int32_t st = check_shape(shape, window);
  if (st != GA_OK) return st;
  if (!std::isfinite(scale)) return GA_ERR_SCALE;
  if (!q || !k_cache || !ctx_lens || !q_pos || !out) return GA_ERR_NULL;
  const bool k_eq_v = v_cache == nullptr || v_cache == k_cache;
  Plan p;
  st = make_plan(shape, window, opts, k_eq_v ? 1 : 0, &p);
  if (st != GA_OK) return st;
  if (p.ws_bytes > (size_t)GA_NOALLOC_SCRATCH_BYTES) return GA_ERR_SCRATCH;
  st = check_arch();
  if (st != GA_OK) return st;
  void* ws = scratch_ptr();
  if (!ws) return GA_ERR_LAUNCH;
  return gemma_attn_decode_ex(shape, q, k_cache, v_cache, ctx_lens, q_pos, window, softcap,
                              scale, out, ws, (size_t)GA_NOALLOC_SCRATCH_BYTES, opts, stream);
}

extern "C" size_t gemma_stream_read_sink_bytes(void) {
  return (size_t)ga::kMaxBlocks * 4 * 64 * 16;
}

extern "C" int32_t gemma_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return GA_ERR_NULL;
  if (!aligned16(src) || !aligned16(sink)) return GA_ERR_NULL;
  if (bytes == 0 || bytes % 1024 != 0) return GA_ERR_DIMS;
  int32_t st = check_arch();
  if (st != GA_OK) return st;
  const hipError_t e =
      ga::stream_read_launch(src, bytes, sink, device_cus(), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GA_OK : GA_ERR_LAUNCH;
}
