/*
 * oracle.c -- fp64 reference for single-token decode attention over bf16 KV caches.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library.  The GPU library never includes, links
 * or calls anything here, and nothing here includes or links the GPU library.
 *
 * What it computes is the plain, unsplit definition of masked softmax attention for
 * one query token per sequence (or T consecutive query tokens per sequence, each with
 * its own causal and window mask), with no blocking, splitting or reordering:
 *
 *   for every batch row b, query token t (at position q_pos = q_pos0_b + t) and query
 *   head h (KV head g = h / G, G = Hq / Hkv):
 *     P  = positions p with 0 <= p <= q_pos, p < ctx, inside the window
 *          (window w > 0: p > q_pos - w) and still present in the cache
 *          (ring of W slots: p >= ctx - W; linear of C slots: p < C)
 *     s_p = scale * <q[b,h,:], K[b,g,slot(p),:]>, then s_p <- c*tanh(s_p/c) when the
 *           soft-cap c is on
 *     out = sum_p softmax(s)_p * V[b,g,slot(p),:],  V = K when no V cache is given
 *     slot(p) = p mod W (ring) or p (linear)
 *
 * Sources (titles and sections of the pages this follows):
 *  - "Gemma support" pull request, Summary: attention logit soft-capping,
 *    sliding-window layers, mixed 256/512 head sizes, K = V global attention.
 *  - "Gemma 4 12B (unified multimodal)" record, KV geometry and "required kernel
 *    class" passages: a local layer reads exactly w KV entries; attention_k_eq_v;
 *    the rotating (ring) cache of sliding layers, in the "(6) On Apple Silicon" item.
 *  - "Gemma4-26B-A4B on Apple Silicon" analysis, Results (Break 4): per-layer-type
 *    head dims and KV-head counts, no separate value projection on full layers;
 *    Threats to validity: the query scale defaults to 1/sqrt(head_dim).
 *  - "Gemma support", Performance: split decode attention (the merge algebra in
 *    oracle_split_merge_f64 is the textbook log-sum-exp identity it rests on); its flash
 *    prefill for head_dim 256 and the spec-decode (k = 7) with sliding-window item of the
 *    "Gemma 4 12B (unified multimodal)" record ("(2)"): several query tokens of one
 *    sequence against the same cache, each masked at its own position.
 * Readings where the pages are silent: the soft-cap is c*tanh(s/c) and is off for
 * c <= 0 or non-finite c; the scale multiplies the raw dot product before the cap;
 * the window is inclusive of the current token and holds exactly w positions; query
 * head h reads KV head h / G; an empty valid set gives out = 0 and lse = -inf.
 *
 * Quantized caches (oracle_decode_fp8_multi_f64): each cached row is D fp8 e4m3 codes
 * (OCP 8-bit float: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, largest finite 448) and one float32 scale; its values are code * scale,
 * and attention is the same definition over those values.  A row is quantized from
 * bf16 as: amax = max |x| (float32), inv = 448 / amax (float32, 0 for amax = 0), code =
 * round-to-nearest-even e4m3 of x * inv (float32 product, clamped to +-448), stored
 * scale = amax / 448 (float32).  Passages: the fp8_e4m3 KV cache and BF16-Q + FP8-KV
 * sliding-window item "(2)" and the rotating quantized cache of item "(6)" of the "Gemma
 * 4 12B (unified multimodal)" record; the per-row dynamic scale is a reading (the pages
 * give no scale granularity).
 *
 * Rotary position embedding (oracle_rope_row): sliding layers use base 10,000 over the
 * whole head, full layers base 1,000,000 applied as a partial rotary to the low part of
 * the head dimension with no positional encoding on the rest ("Gemma support" pull
 * request, Summary: own RoPE base for sliding layers, proportional RoPE; "Gemma 4 12B
 * (unified multimodal)" record, CONTEXT_SCALING_METHOD: rope_type "default" on sliding
 * layers and "proportional" on full layers; "Gemma4-26B-A4B on Apple Silicon", Results
 * (Break 4) and the falsification paragraph: partial rotary on the low portion of the
 * head dimension, nothing on the remainder; the model-loader page's header: bases 10,000
 * and 1,000,000).  With H = D/2 and R (even, <= D) the rotated width: element i and
 * element i + H form rotate-half pair i, which turns by the angle p * base^(-2i/D) for
 * i < R/2; every other element passes through (R = D: the default type, the whole head;
 * R < D: the proportional type, whose frequencies keep the exponent over the whole head
 * and whose rotated pairs are the lowest R/2 of each half).  Computed in double and
 * rounded once to bf16 (round to nearest even).  Pinned against the transformers
 * library's Gemma 4 model code (its rotary embedding for the "default" and "proportional"
 * rope types and its rotate-half application), for both layer types.
 * PARITY UNPINNED: the use of the rotated key row as the value row on K = V layers (one
 * stored row per position is what K = V means here; the pages do not say what the value
 * row is).
 *
 * Arithmetic: every bf16 input is widened exactly (bits << 16 -> float -> double);
 * scale and softcap are widened from their float32 values; libm exp, tanh, log in
 * double.  Results are double; callers round to float32 where they need to.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

/* Precondition flags reported per batch row. */
#define OR_FLAG_QPOS_GE_CTX 1   /* q_pos >= ctx: positions above ctx-1 do not exist   */
#define OR_FLAG_EVICTED 2       /* ring: window or full attention needs evicted slots */
#define OR_FLAG_LINEAR_OVER 4   /* linear: ctx > C, positions >= C do not exist       */
#define OR_FLAG_NEGATIVE 8      /* ctx < 0 or q_pos < 0                               */

enum { OR_LINEAR = 0, OR_RING = 1 };

double oracle_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Membership of position p in the valid set P of one batch row (plain predicate). */
static int in_valid_set(long p, long ctx, long q_pos, long window, int kind, long cap) {
  if (p < 0) return 0;
  if (p > q_pos) return 0;                        /* causal: nothing after the query  */
  if (p > ctx - 1) return 0;                      /* only positions already written   */
  if (window > 0 && p < q_pos - window + 1) return 0; /* exactly w positions up to q */
  if (kind == OR_RING && p < ctx - cap) return 0; /* overwritten in a ring of W slots */
  if (kind == OR_LINEAR && p >= cap) return 0;    /* never stored in a linear cache   */
  return 1;
}

static long slot_of(long p, int kind, long cap) { return kind == OR_RING ? p % cap : p; }

/* Flags for one batch row; 0 when every precondition holds. */
int32_t oracle_row_flags(int32_t ctx, int32_t q_pos, int32_t window, int32_t kind, int32_t cap) {
  int32_t f = 0;
  if (ctx < 0 || q_pos < 0) f |= OR_FLAG_NEGATIVE;
  if (q_pos >= ctx) f |= OR_FLAG_QPOS_GE_CTX;
  if (kind == OR_LINEAR && ctx > cap) f |= OR_FLAG_LINEAR_OVER;
  if (kind == OR_RING) {
    /* oldest position the query wants: q_pos - w + 1 with a window, else 0 */
    long want_lo = window > 0 ? (long)q_pos - window + 1 : 0;
    if (want_lo < 0) want_lo = 0;
    long present_lo = (long)ctx - cap;
    if (want_lo < present_lo && want_lo <= q_pos) f |= OR_FLAG_EVICTED;
  }
  return f;
}

/* Valid set of one batch row: writes the ascending positions and their slots; returns
 * how many there are.  positions/slots may be NULL to only count. */
int64_t oracle_valid_positions(int32_t ctx, int32_t q_pos, int32_t window, int32_t kind,
                               int32_t cap, int64_t* positions, int64_t* slots) {
  int64_t n = 0;
  for (long p = 0; p < (long)ctx; ++p) {
    if (!in_valid_set(p, ctx, q_pos, window, kind, cap)) continue;
    if (positions) positions[n] = p;
    if (slots) slots[n] = slot_of(p, kind, cap);
    ++n;
  }
  return n;
}

typedef struct {
  int B, T, Hq, Hkv, D, cap, kind;
  const uint16_t *q, *k, *v;
  /* fp8 caches (fp8 != 0): codes [B,Hkv,cap,D] and float32 scales [B,Hkv,cap] */
  int fp8;
  const uint8_t *k8, *v8;
  const float *ks, *vs;
  const int32_t *ctx, *qpos;
  int window;
  double softcap; /* <= 0: off */
  double scale;
  double *out, *lse, *probs;
  long probs_len;
  long next_unit;
  pthread_mutex_t mu;
} decode_job;

/* OCP e4m3 (fn) code -> value: exponent field 0 is subnormal (m / 8 * 2^-6); 0x7f and
 * 0xff are NaN; there are no infinities. */
double oracle_e4m3_to_f64(uint8_t c) {
  const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return sgn ? -v : v;
}

/* Round-to-nearest-even of a float32 to e4m3; magnitudes above 448 saturate to +-448
 * (the quantizer clamps before converting, so it never relies on this). */
uint8_t oracle_f32_to_e4m3(float x) {
  const int sgn = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  if (isnan(x)) return 0x7f;
  if (a >= 448.0) return (uint8_t)(sgn | 0x7e);
  if (a < ldexp(1.0, -6)) {  /* subnormal range: multiples of 2^-9 */
    const double q = nearbyint(ldexp(a, 9));  /* 0..8, ties to even */
    return (uint8_t)(sgn | (int)q);           /* q = 8 is 0x08 = 2^-6, the smallest normal */
  }
  int e;
  const double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;                 /* a = (2f) * 2^E, 2f in [1, 2) */
  double m = nearbyint((2.0 * f - 1.0) * 8.0);  /* 0..8, ties to even */
  if (m == 8.0) {
    m = 0.0;
    E += 1;
  }
  return (uint8_t)(sgn | ((E + 7) << 3) | (int)m);
}

/* Round a double to the nearest bf16 (ties to even), directly (no float step, so no
 * double rounding); inputs here are finite and far from the bf16 range limits. */
uint16_t oracle_f64_to_bf16(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  const double f = frexp(fabs(x), &e);       /* |x| = f * 2^e, f in [0.5, 1) */
  const double m = nearbyint(ldexp(f, 8));   /* 8 significant bits, ties to even: 128..256 */
  const float r = (float)ldexp(m, e - 8);    /* exactly representable */
  uint32_t u;
  memcpy(&u, &r, 4);
  return (uint16_t)((u >> 16) | (signbit(x) ? 0x8000 : 0));
}

/* Rotary embedding of one bf16 row x[D] at position p (see header): out_bf16 [D] gets the
 * rounded result, out_f64 [D] (may be NULL) the unrounded one. */
void oracle_rope_row(int D, const uint16_t* x, long p, double base, int R, uint16_t* out_bf16,
                     double* out_f64) {
  const int H = D / 2;
  for (int d = 0; d < D; ++d) {
    double y = oracle_bf16_to_f64(x[d]);
    const int i = d < H ? d : d - H;  /* the pair of element d */
    if (2 * i < R) {
      const double ang = (double)p * pow(base, -2.0 * i / D);
      const double c = cos(ang), s = sin(ang);
      const double a = oracle_bf16_to_f64(x[i]), b = oracle_bf16_to_f64(x[i + H]);
      y = d < H ? a * c - b * s : b * c + a * s;
    }
    if (out_f64) out_f64[d] = y;
    out_bf16[d] = oracle_f64_to_bf16(y);
  }
}

/* Quantize one bf16 row of D values to e4m3 codes and a float32 scale (see header). */
void oracle_quantize_row_fp8(int D, const uint16_t* x, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int d = 0; d < D; ++d) {
    const float v = fabsf((float)oracle_bf16_to_f64(x[d]));
    if (v > amax) amax = v;
  }
  const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
  for (int d = 0; d < D; ++d) {
    float y = (float)oracle_bf16_to_f64(x[d]) * inv;
    y = fminf(fmaxf(y, -448.0f), 448.0f);
    codes[d] = oracle_f32_to_e4m3(y);
  }
  *scale = amax / 448.0f;
}

/* Cached value (row = (b * Hkv + g) * cap + slot, element d) of K (which = 0) or V. */
static double cache_value(const decode_job* J, int which, long row, int d) {
  const long idx = row * J->D + d;
  if (J->fp8) {
    const uint8_t* c = (which == 1 && J->v8) ? J->v8 : J->k8;
    const float* sc = (which == 1 && J->v8) ? J->vs : J->ks;
    return oracle_e4m3_to_f64(c[idx]) * (double)sc[row];
  }
  const uint16_t* c = (which == 1 && J->v) ? J->v : J->k;
  return oracle_bf16_to_f64(c[idx]);
}

/* One query row: unit = (b * T + t) * Hq + h. */
static void decode_unit(decode_job* J, long unit, double* s_buf, long* p_buf) {
  const long bt = unit / J->Hq;
  const int h = (int)(unit % J->Hq);
  const int b = (int)(bt / J->T), t = (int)(bt % J->T);
  const int G = J->Hq / J->Hkv, g = h / G, D = J->D;
  const long ctx = J->ctx[b], qp = (long)J->qpos[b] + t;
  const uint16_t* qrow = J->q + unit * D;
  const long row0 = ((long)b * J->Hkv + g) * (long)J->cap;
  double* orow = J->out + unit * D;

  long n = 0;
  for (long p = 0; p < ctx; ++p)
    if (in_valid_set(p, ctx, qp, J->window, J->kind, J->cap)) p_buf[n++] = p;

  if (J->probs)
    for (long i = 0; i < J->probs_len; ++i) J->probs[unit * J->probs_len + i] = 0.0;
  if (n == 0) {
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (J->lse) J->lse[unit] = -INFINITY;
    return;
  }
  /* logits, in ascending position order */
  for (long i = 0; i < n; ++i) {
    const long krow = row0 + slot_of(p_buf[i], J->kind, J->cap);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += oracle_bf16_to_f64(qrow[d]) * cache_value(J, 0, krow, d);
    double s = J->scale * dot;
    if (J->softcap > 0.0) s = J->softcap * tanh(s / J->softcap);
    s_buf[i] = s;
  }
  double m = s_buf[0];
  for (long i = 1; i < n; ++i)
    if (s_buf[i] > m) m = s_buf[i];
  double l = 0.0;
  for (long i = 0; i < n; ++i) {
    s_buf[i] = exp(s_buf[i] - m);
    l += s_buf[i];
  }
  for (int d = 0; d < D; ++d) orow[d] = 0.0;
  for (long i = 0; i < n; ++i) {
    const long vrow = row0 + slot_of(p_buf[i], J->kind, J->cap);
    const double w = s_buf[i] / l;
    for (int d = 0; d < D; ++d) orow[d] += w * cache_value(J, 1, vrow, d);
    if (J->probs && p_buf[i] < J->probs_len) J->probs[unit * J->probs_len + p_buf[i]] = w;
  }
  if (J->lse) J->lse[unit] = m + log(l);
}

static void* decode_worker(void* arg) {
  decode_job* J = (decode_job*)arg;
  long maxctx = 1;
  for (int b = 0; b < J->B; ++b)
    if (J->ctx[b] > maxctx) maxctx = J->ctx[b];
  double* s_buf = (double*)malloc(sizeof(double) * maxctx);
  long* p_buf = (long*)malloc(sizeof(long) * maxctx);
  if (!s_buf || !p_buf) {
    free(s_buf);
    free(p_buf);
    return (void*)1;
  }
  const long units = (long)J->B * J->T * J->Hq;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    long u = J->next_unit++;
    pthread_mutex_unlock(&J->mu);
    if (u >= units) break;
    decode_unit(J, u, s_buf, p_buf);
  }
  free(s_buf);
  free(p_buf);
  return NULL;
}

int oracle_num_threads_default(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static int run_decode(decode_job* J, const int32_t* ctx_lens, const int32_t* q_pos0, int window,
                      float softcap, float scale, int32_t* flags, int nthreads) {
  const int B = J->B, T = J->T, Hq = J->Hq;
  if (flags)
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < T; ++t)
        flags[(long)b * T + t] = oracle_row_flags(ctx_lens[b], q_pos0[b] + t, window, J->kind,
                                                  J->cap);
  J->ctx = ctx_lens;
  J->qpos = q_pos0;
  J->window = window;
  J->softcap = (isfinite(softcap) && softcap > 0.0f) ? (double)softcap : 0.0;
  J->scale = (double)scale;
  J->next_unit = 0;
  pthread_mutex_init(&J->mu, NULL);
  if (nthreads <= 0) nthreads = oracle_num_threads_default();
  long units = (long)B * T * Hq;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  if (!th) return OR_ENOMEM;
  int rc = OR_OK;
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, decode_worker, J);
  for (int i = 0; i < nthreads; ++i) {
    void* r = NULL;
    pthread_join(th[i], &r);
    if (r) rc = OR_ENOMEM;
  }
  free(th);
  pthread_mutex_destroy(&J->mu);
  return rc;
}

/*
 * Decode attention for every (b, t, h) with T query tokens per batch row.  q [B,T,Hq,D];
 * k_cache and v_cache [B,Hkv,cap,D] (bf16 bits, contiguous); v_cache NULL means V = K;
 * q_pos0 [B] is the position of token 0, token t sits at q_pos0[b] + t.  out [B,T,Hq,D]
 * double; lse [B*T*Hq] (may be NULL); probs [B*T*Hq, probs_len] indexed by absolute
 * position (may be NULL); flags [B*T] receives each token's precondition flags (may be
 * NULL).  nthreads <= 0: all cores.  Returns 0, or OR_EINVAL / OR_ENOMEM.
 */
int oracle_decode_multi_f64(int B, int T, int Hq, int Hkv, int D, int cap, int kind,
                            const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* ctx_lens, const int32_t* q_pos0, int window,
                            float softcap, float scale, double* out, double* lse, double* probs,
                            long probs_len, int32_t* flags, int nthreads) {
  if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || cap <= 0 || Hq % Hkv != 0)
    return OR_EINVAL;
  if (kind != OR_LINEAR && kind != OR_RING) return OR_EINVAL;
  if (!q || !k_cache || !ctx_lens || !q_pos0 || !out) return OR_EINVAL;
  if (!isfinite(scale)) return OR_EINVAL;
  decode_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.cap = cap; J.kind = kind;
  J.q = q; J.k = k_cache; J.v = v_cache;
  J.out = out; J.lse = lse; J.probs = probs; J.probs_len = probs ? probs_len : 0;
  return run_decode(&J, ctx_lens, q_pos0, window, softcap, scale, flags, nthreads);
}

/*
 * oracle_decode_multi_f64 over fp8 caches: k_codes [B,Hkv,cap,D] e4m3 codes with
 * k_scales [B,Hkv,cap] float32, V likewise, or v_codes NULL for K = V.  Each cached
 * value is code * scale (exact in double); the rest is the same definition.
 */
int oracle_decode_fp8_multi_f64(int B, int T, int Hq, int Hkv, int D, int cap, int kind,
                                const uint16_t* q, const uint8_t* k_codes, const float* k_scales,
                                const uint8_t* v_codes, const float* v_scales,
                                const int32_t* ctx_lens, const int32_t* q_pos0, int window,
                                float softcap, float scale, double* out, double* lse,
                                double* probs, long probs_len, int32_t* flags, int nthreads) {
  if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || cap <= 0 || Hq % Hkv != 0)
    return OR_EINVAL;
  if (kind != OR_LINEAR && kind != OR_RING) return OR_EINVAL;
  if (!q || !k_codes || !k_scales || !ctx_lens || !q_pos0 || !out) return OR_EINVAL;
  if ((v_codes == NULL) != (v_scales == NULL)) return OR_EINVAL;
  if (!isfinite(scale)) return OR_EINVAL;
  decode_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.cap = cap; J.kind = kind;
  J.q = q; J.fp8 = 1; J.k8 = k_codes; J.ks = k_scales; J.v8 = v_codes; J.vs = v_scales;
  J.out = out; J.lse = lse; J.probs = probs; J.probs_len = probs ? probs_len : 0;
  return run_decode(&J, ctx_lens, q_pos0, window, softcap, scale, flags, nthreads);
}

/*
 * Quantizing append of T tokens per row into an fp8 cache: token t of row b (new_rows
 * [B,T,Hkv,D] bf16) goes to position pos0[b] + t, slot p mod W (ring) or p (linear), in
 * order t = 0..T-1; positions that are negative or (linear) >= C are skipped.
 */
int oracle_append_fp8(int B, int T, int Hkv, int D, int cap, int kind, uint8_t* codes,
                      float* scales, const uint16_t* new_rows, const int32_t* pos0) {
  if (B < 0 || T <= 0 || Hkv <= 0 || D <= 0 || cap <= 0 || !codes || !scales || !new_rows ||
      !pos0)
    return OR_EINVAL;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t) {
      const long p = (long)pos0[b] + t;
      if (p < 0 || (kind == OR_LINEAR && p >= cap)) continue;
      const long s = slot_of(p, kind, cap);
      for (int g = 0; g < Hkv; ++g) {
        const long row = ((long)b * Hkv + g) * cap + s;
        oracle_quantize_row_fp8(D, new_rows + (((long)b * T + t) * Hkv + g) * D,
                                codes + row * D, scales + row);
      }
    }
  return OR_OK;
}

/*
 * Decode attention for every (b, h), one query token per row at q_pos[b]: the T = 1
 * case of oracle_decode_multi_f64.  q [B,Hq,D]; out [B,Hq,D]; lse [B*Hq]; flags [B].
 */
int oracle_decode_f64(int B, int Hq, int Hkv, int D, int cap, int kind, const uint16_t* q,
                      const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* ctx_lens,
                      const int32_t* q_pos, int window, float softcap, float scale, double* out,
                      double* lse, double* probs, long probs_len, int32_t* flags, int nthreads) {
  return oracle_decode_multi_f64(B, 1, Hq, Hkv, D, cap, kind, q, k_cache, v_cache, ctx_lens,
                                 q_pos, window, softcap, scale, out, lse, probs, probs_len, flags,
                                 nthreads);
}

/*
 * Cache append: cache[b, g, slot(pos_b), :] <- new[b, g, :] for every (b, g), with
 * slot(p) = p mod W (ring) or p (linear).  new [B,Hkv,D]; cache [B,Hkv,cap,D].
 * Returns OR_EINVAL for a negative position or a linear position >= C.
 */
int oracle_append(int B, int Hkv, int D, int cap, int kind, uint16_t* cache, const uint16_t* new_rows,
                  const int32_t* pos) {
  if (B < 0 || Hkv <= 0 || D <= 0 || cap <= 0 || !cache || !new_rows || !pos) return OR_EINVAL;
  for (int b = 0; b < B; ++b) {
    if (pos[b] < 0 || (kind == OR_LINEAR && pos[b] >= cap)) return OR_EINVAL;
  }
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      long s = slot_of(pos[b], kind, cap);
      uint16_t* dst = cache + (((long)b * Hkv + g) * cap + s) * D;
      const uint16_t* src = new_rows + ((long)b * Hkv + g) * D;
      for (int d = 0; d < D; ++d) dst[d] = src[d];
    }
  return OR_OK;
}

/*
 * Split-and-merge in fp64 for ONE query row, used only to pin the merge algebra.
 * logits [n] (already scaled and capped), values [n, D] (double), a partition of
 * 0..n-1 into nparts consecutive pieces given by cut points starts[0..nparts]
 * (starts[0] = 0, starts[nparts] = n; an empty piece is allowed).  Each piece yields
 * (m_s, l_s, acc_s) with m_s = max, l_s = sum exp(s - m_s), acc_s = sum exp(s - m_s) v;
 * the merge is M = max m_s, L = sum l_s e^{m_s - M}, out = sum e^{m_s - M} acc_s / L.
 * An empty piece has m = -inf, l = 0, acc = 0 and contributes nothing.  out [D];
 * returns lse = M + log L (-inf when n = 0, and then out = 0).
 */
double oracle_split_merge_f64(long n, int D, const double* logits, const double* values, int nparts,
                              const long* starts, double* out) {
  double M = -INFINITY;
  double* ms = (double*)malloc(sizeof(double) * (nparts > 0 ? nparts : 1));
  double* ls = (double*)malloc(sizeof(double) * (nparts > 0 ? nparts : 1));
  double* accs = (double*)calloc((size_t)(nparts > 0 ? nparts : 1) * D, sizeof(double));
  for (int s = 0; s < nparts; ++s) {
    double m = -INFINITY, l = 0.0;
    for (long i = starts[s]; i < starts[s + 1]; ++i)
      if (logits[i] > m) m = logits[i];
    for (long i = starts[s]; i < starts[s + 1]; ++i) {
      double e = exp(logits[i] - m);
      l += e;
      for (int d = 0; d < D; ++d) accs[(long)s * D + d] += e * values[i * D + d];
    }
    ms[s] = m;
    ls[s] = l;
    if (m > M) M = m;
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  double L = 0.0;
  if (M == -INFINITY) {
    free(ms); free(ls); free(accs);
    return -INFINITY;
  }
  for (int s = 0; s < nparts; ++s) {
    if (ls[s] == 0.0) continue;
    double f = exp(ms[s] - M);
    L += ls[s] * f;
    for (int d = 0; d < D; ++d) out[d] += f * accs[(long)s * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= L;
  free(ms); free(ls); free(accs);
  (void)n;
  return M + log(L);
}
