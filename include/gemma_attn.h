/*
 * gemma_attn.h -- single-token decode attention for hybrid sliding/global stacks on
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and status codes.
 *
 * What is computed (one query token per sequence, per layer):
 *   for batch row b, query head h, KV head g = h / G with G = Hq / Hkv:
 *     valid positions P_b = { p : max(lo_w, lo_ring, 0) <= p <= min(q_pos_b, ctx_b - 1) }
 *       lo_w    = q_pos_b - window + 1 when window > 0 (exactly `window` positions,
 *                 the current one included), else 0 (full causal);
 *       lo_ring = ctx_b - W for a ring cache of W slots (older entries are overwritten)
 *     s_p  = scale * dot(q[b,h,:], K[b,g,slot(p),:])        (fp32 accumulation)
 *     s_p <- softcap * tanh(s_p / softcap)   when 0 < softcap < inf
 *     out[b,h,:] = sum_p softmax(s)_p * V[b,g,slot(p),:]    (V = K when K = V)
 *     slot(p) = p mod W (ring) or p (linear); an empty P_b gives out = 0.
 *   Passages defining the operation (page titles and sections):
 *     - "Gemma support" pull request, Summary: attention logit soft-capping,
 *       sliding-window layers, mixed 256/512 head sizes, K = V global attention;
 *       Performance: split decode attention for head sizes 256/512; Test plan:
 *       kernel tests over head sizes 128 to 512 (hence head_dim 128 is accepted too).
 *     - "Gemma 4 12B (unified multimodal)" record: a local layer reads exactly w KV
 *       entries ("required kernel class"); per-layer-type cache management; the
 *       rotating (ring) KV cache of sliding layers ("(6) On Apple Silicon");
 *       attention_k_eq_v; head_dim 256 / 8 KV heads sliding, 512 / 1 KV head global.
 *     - "Gemma4-26B-A4B on Apple Silicon", Results (Break 4): K/V sharing on full
 *       layers, no separate value projection; Threats to validity: query scale
 *       defaults to 1/sqrt(head_dim).
 *     - same record, "(4) On Hopper": one KV head and batch 1 cannot fill a GPU
 *       without splitting the keys, which is why the keys are split across CUs and
 *       merged by log-sum-exp.
 *
 * Layout (all contiguous, row-major, bf16 as raw uint16 bits):
 *   q        [B, Hq, D]          out [B, Hq, D] float32
 *   caches   [B, Hkv, capacity, D]   (head-major: each (b, g) is one run of rows)
 *   ctx_lens, q_pos, pos: int32 [B] in DEVICE memory
 * Every pointer except the shape/opts structs is a device pointer.
 *
 * Ownership and execution: the caller owns every buffer.  The library keeps no
 * pointer after a call returns, never allocates, frees or synchronises device memory,
 * and enqueues all work on `stream` (a hipStream_t; NULL = the default stream).  Calls
 * return as soon as the work is enqueued.  The only state kept is a per-device cache
 * of the architecture check.
 *
 * Errors: every entry point returns int32_t, GA_OK (0) or a negative GA_ERR_* code
 * (gemma_attn_strerror names it).  Arguments are checked on the host before anything
 * is launched; on error nothing is launched.  Nothing throws across the ABI.
 * Preconditions on device data (0 <= q_pos < ctx; linear: ctx <= C; ring: the window's
 * positions are still present, q_pos - window + 1 >= ctx - W) belong to the caller:
 * the kernels clamp every index so a violation never reads or writes out of bounds,
 * and gemma_attn_validate reports it.
 */
#ifndef GEMMA_ATTN_H
#define GEMMA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t ga_bf16; /* raw bf16 bits */

enum { GA_CACHE_LINEAR = 0, GA_CACHE_RING = 1 };

/* Status codes. */
enum {
  GA_OK = 0,
  GA_ERR_NULL = -1,          /* a required pointer is NULL                                */
  GA_ERR_DIMS = -2,          /* batch < 0, a head count or capacity <= 0                  */
  GA_ERR_HEAD_DIM = -3,      /* head_dim is not 128, 256 or 512                           */
  GA_ERR_GQA = -4,           /* num_q_heads is not a multiple of num_kv_heads, or G > 16  */
  GA_ERR_KIND = -5,          /* kind is neither GA_CACHE_LINEAR nor GA_CACHE_RING         */
  GA_ERR_WINDOW = -6,        /* ring: window > W, or window <= 0 while max_ctx may exceed W,
                                or (multi-token) window + T - 1 > W while it may           */
  GA_ERR_WORKSPACE = -7,     /* workspace NULL or smaller than ga_decode_workspace_bytes  */
  GA_ERR_SCALE = -8,         /* scale is not finite                                       */
  GA_ERR_V_MISMATCH = -9,    /* exactly one of v_cache / v_new is NULL                    */
  GA_ERR_ARCH = -10,         /* no device, or the current device is not gfx950            */
  GA_ERR_LAUNCH = -11,       /* a kernel launch failed (hipGetLastError)                  */
  GA_ERR_OPTS = -12,         /* decode options out of range or not valid for this shape   */
  GA_ERR_MAX_CTX = -13,      /* max_ctx < 0, or linear max_ctx > capacity                 */
  GA_ERR_TOO_LARGE = -14,    /* a size overflows the 32-bit grid or index arithmetic      */
  GA_ERR_SCRATCH = -15       /* gemma_attn_decode_noalloc: the call needs more workspace
                                than its fixed device scratch holds                       */
};

/* Shape of one layer's decode call. */
typedef struct ga_shape {
  int32_t batch;        /* B >= 0 (0: nothing to do)                                  */
  int32_t num_q_heads;  /* Hq > 0                                                     */
  int32_t num_kv_heads; /* Hkv > 0, Hq % Hkv == 0, G = Hq / Hkv <= 16                 */
  int32_t head_dim;     /* D: 128, 256 or 512                                         */
  int32_t capacity;     /* ring: W slots; linear: C positions                         */
  int32_t kind;         /* GA_CACHE_LINEAR or GA_CACHE_RING                           */
  int32_t max_ctx;      /* host upper bound on every ctx_lens[b]; 0 means `capacity`  */
} ga_shape;

/* Implementation choice for the split kernel. */
enum { GA_IMPL_AUTO = 0, GA_IMPL_VALU = 1, GA_IMPL_MFMA = 2 };

/* Optional decode options (NULL = all automatic). */
typedef struct ga_decode_opts {
  int32_t split_keys; /* keys per split work unit: 0 = automatic; otherwise a multiple
                         of 64 in [64, 65536].  Results are split-invariant within
                         rounding.                                                     */
  int32_t impl;       /* GA_IMPL_*; MFMA exists for head_dim 512 with G = 16 and K = V */
  int32_t deterministic; /* 1: the vector kernel visits keys in a fixed order, so repeated
                            calls give identical bits; 0 (default): keys are handed to
                            waves dynamically, which is faster and equal within rounding */
  int32_t reserved[5]; /* must be zero                                                 */
} ga_decode_opts;

/*
 * Bytes of device workspace gemma_attn_decode needs for this shape, window and options.
 * Vector path: split partials in fp32, acc [B, Hq, S, D] then (m, l) [B, Hq, S, 2], with
 * S the host upper bound of splits per row; 0 when every row fits in one split (no
 * workspace is touched).  Matrix-core path (head_dim 512, 16 query heads per KV head,
 * K = V): one launch covers at most 1024 units (B * Hkv, whole rows; larger batches run
 * as several launches that reuse the workspace), and each of its P work-groups writes
 * one partial, acc [P, 16, 512] then (m, l) [P, 16, 2] in fp32, followed by the per-unit
 * work-group prefix sums [U + 1] int32 (U units in one launch).  Without a split size
 * P = N when U <= 3N/4 and N + U otherwise, N = 256 (a call on a device with fewer
 * compute units uses that count and needs less); with a split size of s keys,
 * P = U * ceil(Kmax / round_up(s, 64)), Kmax the largest key count any row can see.
 * When the query cannot tell which path a call will take (GA_IMPL_AUTO and the
 * matrix-core geometry, K = V not known), the maximum of both.  Returns SIZE_MAX when
 * the arguments are invalid (the decode call would fail).
 */
size_t ga_decode_workspace_bytes(const ga_shape* shape, int32_t window, const ga_decode_opts* opts);

/*
 * Single-token decode attention (see the definition above).
 *   q        device bf16 [B, Hq, D]
 *   k_cache  device bf16 [B, Hkv, capacity, D]
 *   v_cache  device bf16, same shape, or NULL when K = V (the K tensor is read once per
 *            tile and used as both keys and values)
 *   ctx_lens device int32 [B]: positions 0..ctx-1 have been appended
 *   q_pos    device int32 [B]: absolute position of the query token (usually ctx - 1)
 *   window   > 0: sliding window of `window` positions; <= 0: full causal
 *   softcap  > 0 and finite: tanh soft-cap of the scaled logits; otherwise off
 *   scale    finite query scale applied to the fp32 dot products
 *   out      device float32 [B, Hq, D], fully overwritten
 *   workspace/workspace_bytes  device scratch of at least ga_decode_workspace_bytes
 *            (may be NULL when that is 0); contents need not be initialised
 * Launches the split kernel and, when any row can need more than one split, the
 * log-sum-exp merge kernel, both on `stream`.
 */
int32_t gemma_attn_decode(const ga_shape* shape, const ga_bf16* q, const ga_bf16* k_cache,
                          const ga_bf16* v_cache, const int32_t* ctx_lens, const int32_t* q_pos,
                          int32_t window, float softcap, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* gemma_attn_decode with explicit options (split size, implementation); opts may be NULL. */
int32_t gemma_attn_decode_ex(const ga_shape* shape, const ga_bf16* q, const ga_bf16* k_cache,
                             const ga_bf16* v_cache, const int32_t* ctx_lens, const int32_t* q_pos,
                             int32_t window, float softcap, float scale, float* out, void* workspace,
                             size_t workspace_bytes, const ga_decode_opts* opts, void* stream);

/*
 * Cache append fused with decode, in one launch: exactly gemma_kv_append(shape, k_cache,
 * v_cache, k_new, v_new, pos) followed by gemma_attn_decode_ex(...) on the same stream,
 * bit for bit (cache contents and output).  One work-group per (b, g) writes the new row;
 * every key whose slot is the appended slot is read from k_new / v_new instead of the
 * cache, so no work-group reads a slot while it is being written.  Arguments as in the
 * two calls; k_new [B, Hkv, D] and pos [B] device pointers must be non-NULL, and v_new is
 * NULL exactly when v_cache is (K = V).  Saves the separate append launch per layer.
 */
int32_t gemma_attn_decode_append(const ga_shape* shape, const ga_bf16* q, ga_bf16* k_cache,
                                 ga_bf16* v_cache, const ga_bf16* k_new, const ga_bf16* v_new,
                                 const int32_t* pos, const int32_t* ctx_lens,
                                 const int32_t* q_pos, int32_t window, float softcap, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 const ga_decode_opts* opts, void* stream);

/*
 * Cache append of one token per sequence: cache[b, g, slot(pos_b), :] <- new[b, g, :]
 * for K, and for V unless K = V.  Ring: slot = pos mod W; linear: slot = pos.
 *   k_new, v_new device bf16 [B, Hkv, D]; v_cache and v_new are both NULL for K = V.
 *   pos device int32 [B]: absolute position of the new token (>= 0; linear: < C).
 * A row whose position is out of range (negative, or >= C for linear) is skipped:
 * nothing is written for it.  The copy is bit-exact.
 * Passages: "Gemma 4 12B (unified multimodal)" record, per-layer-type cache management
 * and the rotating KV cache of sliding layers; "gemma-4-E2B-CoreAI" model card,
 * the KV cache that grows on the device during decode.
 */
int32_t gemma_kv_append(const ga_shape* shape, ga_bf16* k_cache, ga_bf16* v_cache,
                        const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                        void* stream);

/*
 * Multi-token decode: T = num_tokens consecutive query tokens per sequence (speculative
 * verification of T - 1 draft tokens, or a chunk of prefill) against the same cache,
 * each token masked at its own position.  Token t of row b sits at position
 * q_pos[b] + t and attends to the positions p with
 *     max(0, q_pos[b] + t - window + 1 [window > 0], ctx_b - W [ring]) <= p
 *     p <= min(q_pos[b] + t, ctx_b - 1)      (linear also p < C),
 * i.e. exactly the single-token definition applied per token.  Passages: "Gemma
 * support" pull request, Performance (flash prefill for head_dim 256, split decode) and
 * the spec-decode (k = 7) with sliding-window item "(2)" of the "Gemma 4 12B (unified
 * multimodal)" record, where a kernel mis-selected the window's keys at some
 * seq_len / page alignments.
 *   q        device bf16 [B, T, Hq, D]        out  device float32 [B, T, Hq, D]
 *   q_pos    device int32 [B]: position of token 0 (usually ctx - T after appending)
 *   other arguments as in gemma_attn_decode_ex (GA_IMPL_MFMA is not offered here).
 * Ring caches: when the context can exceed W (max_ctx > W) the ring must keep
 * window + T - 1 slots (token 0's window begins T - 1 positions before token T-1's);
 * a smaller ring is refused with GA_ERR_WINDOW.  Work: each unit (b, KV head, chunk of
 * tokens) reads the union of its tokens' key ranges once.  T = 1 is gemma_attn_decode_ex.
 */
size_t ga_decode_multi_workspace_bytes(const ga_shape* shape, int32_t num_tokens, int32_t window,
                                       const ga_decode_opts* opts);
int32_t gemma_attn_decode_multi(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                                const ga_bf16* k_cache, const ga_bf16* v_cache,
                                const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                                float softcap, float scale, float* out, void* workspace,
                                size_t workspace_bytes, const ga_decode_opts* opts, void* stream);

/*
 * Append of T = num_tokens tokens per sequence at positions pos[b] + t, t = 0..T-1, in
 * that order (when two tokens land in the same ring slot the later one stays).
 *   k_new, v_new device bf16 [B, T, Hkv, D]; pos device int32 [B].
 * Out-of-range positions are skipped, as in gemma_kv_append (its T = 1 case).
 */
int32_t gemma_kv_append_multi(const ga_shape* shape, int32_t num_tokens, ga_bf16* k_cache,
                              ga_bf16* v_cache, const ga_bf16* k_new, const ga_bf16* v_new,
                              const int32_t* pos, void* stream);

/*
 * Quantized (fp8) caches: each cached row is D e4m3 codes (OCP 8-bit float: 4 exponent
 * bits with bias 7, 3 mantissa bits, largest finite 448, no infinities) plus one float32
 * scale, and stands for the values code * scale.  Half the bytes of a bf16 cache per
 * key.  Passages: the fp8_e4m3 KV cache (BF16 queries with FP8 KV on sliding-window
 * layers, item "(2)") and the rotating quantized cache (item "(6)") of the "Gemma 4 12B
 * (unified multimodal)" record.  The per-row scale is this library's choice.
 *   k_codes  device uint8 [B, Hkv, capacity, D] (16-byte aligned)
 *   k_scales device float32 [B, Hkv, capacity]
 *   v_codes / v_scales  the same for V, or both NULL for K = V
 *
 * Quantizing append of T = num_tokens tokens per row (T = 1: one token), at positions
 * pos[b] + t in order t = 0..T-1 (a later token landing in the same ring slot stays;
 * out-of-range positions are skipped).  For each new row x (bf16 [D]): amax = max |x|,
 * inv = 448 / amax (0 when amax = 0), code_d = round-to-nearest-even e4m3 of
 * clamp(x_d * inv, -448, 448), scale = amax / 448, in float32 with correctly rounded
 * division.  k_new, v_new: device bf16 [B, T, Hkv, D]; v_* NULL for K = V.
 */
int32_t gemma_kv_append_fp8(const ga_shape* shape, int32_t num_tokens, uint8_t* k_codes,
                            float* k_scales, uint8_t* v_codes, float* v_scales,
                            const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                            void* stream);

/*
 * Decode over fp8 caches: T = num_tokens query tokens per row (q [B, T, Hq, D], out
 * [B, T, Hq, D], token t at q_pos[b] + t; T = 1 is single-token decode with q [B, Hq, D]).
 * Same definition, with every cached value code * scale; the logits accumulate
 * q . codes in float32 and multiply by the row's K scale, the value weights carry the
 * row's V scale.  The kernels are chosen as for bf16 caches: with one token, the K = V
 * global geometry (head_dim 512, 16 query heads per KV head) runs on the matrix cores;
 * with several tokens, 16 query rows per KV head (heads x tokens >= 4, padded to 16;
 * head_dim 128 or 256, or 512 with K = V) run on the matrix cores; there the codes are
 * widened exactly to bf16 (every e4m3 value is a bf16 value), the K scale multiplies
 * each logit and the V scale each value weight.  Every other shape runs on the vector
 * kernel (GA_IMPL_MFMA is refused there).
 * Workspace: ga_decode_fp8_workspace_bytes (covers whichever kernel the call picks).
 */
size_t ga_decode_fp8_workspace_bytes(const ga_shape* shape, int32_t num_tokens, int32_t window,
                                     const ga_decode_opts* opts);
int32_t gemma_attn_decode_fp8(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                              const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales,
                              const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                              float softcap, float scale, float* out, void* workspace,
                              size_t workspace_bytes, const ga_decode_opts* opts, void* stream);

/*
 * Quantizing append of one token fused with single-token decode over fp8 caches: exactly
 * gemma_kv_append_fp8(shape, 1, k_codes, k_scales, v_codes, v_scales, k_new, v_new, pos)
 * followed by gemma_attn_decode_fp8(shape, 1, q, k_codes, k_scales, v_codes, v_scales,
 * ctx_lens, q_pos, ...), bit for bit (codes, scales and out).  Where the vector kernel
 * serves the call (the sliding geometry), one launch does both: one wave of each
 * work-group quantizes the new rows with the append's own arithmetic, every reader of the
 * appended slot takes those codes and scales from registers, and the first split stores
 * them.  The matrix-core kernel of the K = V global geometry does the same in its one
 * launch: every work-group quantizes its unit's new row, the unit's first work-group stores
 * it, and the wave whose step holds the appended key puts the new codes (widened) and scale
 * in place of what it loaded from the slot.
 * k_new, v_new [B, Hkv, D] device bf16 (v_new NULL exactly when v_codes is, K = V) and
 * pos [B] device int32, non-NULL; other arguments and errors as in the two calls;
 * workspace: ga_decode_fp8_workspace_bytes(shape, 1, window, opts).
 */
int32_t gemma_attn_decode_append_fp8(const ga_shape* shape, const ga_bf16* q, uint8_t* k_codes,
                                     float* k_scales, uint8_t* v_codes, float* v_scales,
                                     const ga_bf16* k_new, const ga_bf16* v_new,
                                     const int32_t* pos, const int32_t* ctx_lens,
                                     const int32_t* q_pos, int32_t window, float softcap,
                                     float scale, float* out, void* workspace,
                                     size_t workspace_bytes, const ga_decode_opts* opts,
                                     void* stream);

/*
 * cos / sin table of the rotary embedding of one token per row, at position pos[b]:
 *   table[b, i, 0] = cos(pos[b] * rope_base^(-2i/D)), table[b, i, 1] = sin(...)
 * for the R / 2 turning rotate-half pairs i of R = rotary_dim and D = head_dim (definition
 * at gemma_rope_append), computed in double by the same function as gemma_rope_append's
 * angles, so the two give the same bits.  The angles depend on the position, the base, R
 * and D only, so a decode step computes one table per layer type (all sliding layers share
 * one base, R and D, all global layers another: "Gemma support" pull request, Summary) and
 * every layer of that type reads it.  table: device float64 [batch, R / 2, 2], 16-byte
 * aligned, fully written.  pos: device int32 [batch].  Errors: GA_ERR_DIMS (batch < 0, R
 * odd, negative or above head_dim), GA_ERR_HEAD_DIM (head_dim not 128, 256 or 512),
 * GA_ERR_OPTS (rope_base not finite and > 0), GA_ERR_NULL.  Nothing is launched when batch
 * or R is 0.
 */
int32_t gemma_rope_table(int32_t batch, const int32_t* pos, float rope_base, int32_t rotary_dim,
                         int32_t head_dim, double* table, void* stream);

/*
 * RoPE, cache append and single-token decode in one call: exactly
 *   gemma_rope_append(shape, 1, q, q_out, k_cache, v_cache, k_new, v_new, pos, rope_base,
 *                     rotary_dim, stream)
 * followed by gemma_attn_decode_ex(shape, q_out, k_cache, v_cache, ctx_lens, q_pos, window,
 * softcap, scale, out, workspace, workspace_bytes, opts, stream), bit for bit (q_out, the
 * caches and out), where rope_table is gemma_rope_table(B, pos, rope_base, rotary_dim,
 * shape->head_dim).
 * q [B, Hq, D] and k_new [B, Hkv, D] are rotated at position pos[b]; v_new is appended
 * unrotated, NULL with v_cache for K = V (the one stored row is then the rotated key, and
 * the values are read from it as well).  q_out [B, Hq, D] device bf16, non-NULL, 16-byte
 * aligned; it may equal q and must not otherwise overlap it.  rope_table as written by
 * gemma_rope_table (may be NULL when rotary_dim is 0).  Workspace: ga_decode_workspace_bytes,
 * as for the decode.  Where the vector kernel serves the call, one launch does it all (the
 * sliding layers: head_dim 256 with their own RoPE base, "Gemma support" pull request,
 * Summary; 8 KV heads under 16 query heads, "Gemma 4 12B (unified multimodal)" record, KV
 * geometry): each work-group rotates
 * its unit's query rows and the new K row into LDS, the first split writes the rotated q
 * and appends the rotated row, and every reader of the appended slot takes the rotated row
 * from LDS; with q_out == q that needs a single split per row.  The matrix-core kernel
 * of the K = V global geometry (partial rotary on its low dimensions, "Gemma4-26B-A4B on
 * Apple Silicon ... (NO-GO)", Results, Break 4) does the same in its one launch when
 * q_out is a separate buffer.  Otherwise (an in-place q_out with several splits, the
 * multi-token matrix-core kernel) the RoPE + append kernel runs first, on the table's
 * angles, then the decode.  Errors: those of both calls (GA_ERR_OPTS for rotary_dim),
 * checked before anything is launched.
 */
int32_t gemma_attn_decode_rope_append(const ga_shape* shape, const ga_bf16* q, ga_bf16* q_out,
                                      ga_bf16* k_cache, ga_bf16* v_cache, const ga_bf16* k_new,
                                      const ga_bf16* v_new, const int32_t* pos,
                                      const int32_t* ctx_lens, const int32_t* q_pos,
                                      int32_t window, float softcap, float scale,
                                      const double* rope_table, int32_t rotary_dim, float* out,
                                      void* workspace, size_t workspace_bytes,
                                      const ga_decode_opts* opts, void* stream);

/*
 * Rotary position embedding fused with the cache append, one launch for T = num_tokens
 * tokens per row at positions pos[b] + t (T = 1: decode):
 *   q_out[b,t,h,:] = rope(q[b,t,h,:], pos[b] + t)            (q, q_out [B, T, Hq, D])
 *   k_cache[b,g,slot(pos[b]+t),:] = rope(k_new[b,t,g,:], ...) (k_new [B, T, Hkv, D])
 *   v_cache[...] = v_new[b,t,g,:] unrotated (v_cache and v_new NULL for K = V, whose one
 *   cached row is the rotated key, read as the value row too)
 * rope(x, p): elements i and i + D/2 form rotate-half pair i; for i < R/2 (R = rotary_dim,
 * even, 0 <= R <= D) the pair turns by the angle p * rope_base^(-2i/D), and every other
 * element passes through.  Sliding layers: base 10,000, R = D (the whole head, rope_type
 * default); full layers: base 1,000,000, R = D/4 (rope_type proportional: the lowest
 * quarter of the pairs turn, their frequencies still over the whole head) ("Gemma support"
 * pull request, Summary: own RoPE base for sliding layers, proportional RoPE; "Gemma 4 12B
 * (unified multimodal)" record, CONTEXT_SCALING_METHOD: the rope types per layer type;
 * "Gemma4-26B-A4B on Apple Silicon", Results (Break 4): partial rotary on the low portion
 * of full-attention heads).  Computed in double, rounded once to bf16 (nearest, ties to
 * even).  q_out may equal q (in place).  Append rules as in gemma_kv_append_multi
 * (out-of-range positions skipped; the latest token owns a shared ring slot).  One pass
 * over q and the new rows replaces a rotary pass plus an append pass.  k_cache, k_new,
 * v_cache and v_new all NULL rotates q only (a layer that reads another layer's cache).
 */
int32_t gemma_rope_append(const ga_shape* shape, int32_t num_tokens, const ga_bf16* q,
                          ga_bf16* q_out, ga_bf16* k_cache, ga_bf16* v_cache,
                          const ga_bf16* k_new, const ga_bf16* v_new, const int32_t* pos,
                          float rope_base, int32_t rotary_dim, void* stream);

/*
 * Allocation-free single-token decode, for callers that cannot allocate device memory or
 * manage a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): exactly gemma_attn_decode_ex(shape, q, k_cache, v_cache, ctx_lens,
 * q_pos, window, softcap, scale, out, <scratch>, GA_NOALLOC_SCRATCH_BYTES, opts, stream),
 * same kernels and same results, with the library's own device scratch as the workspace.
 * The scratch is a fixed array of GA_NOALLOC_SCRATCH_BYTES in device memory, one per
 * device the library runs on, held until the process ends; the call itself allocates and
 * frees nothing.  A call whose workspace (ga_decode_workspace_bytes for the same shape,
 * window and options) exceeds it returns GA_ERR_SCRATCH with nothing launched.  32 MiB
 * holds 1020 partials of the global matrix-core path (its balanced partition for up to 764
 * units of batch rows x KV heads; the Gemma-4-12B global layer at batch 16 needs 8.4 MB)
 * and the vector path's split partials up to the same size.  Every call on one device
 * shares that device's scratch: calls that overlap in time on one device (on different
 * streams, or from different threads without ordering) race on it and must not be issued;
 * calls ordered on one stream are safe.  Other arguments, ownership and errors as for
 * gemma_attn_decode_ex.
 */
#define GA_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t gemma_attn_decode_noalloc(const ga_shape* shape, const ga_bf16* q, const ga_bf16* k_cache,
                                  const ga_bf16* v_cache, const int32_t* ctx_lens,
                                  const int32_t* q_pos, int32_t window, float softcap,
                                  float scale, float* out, const ga_decode_opts* opts,
                                  void* stream);

/*
 * Measurement aid: the practical read ceiling the decode kernels are measured against.
 * Decode attention is bound by streaming the cache ("Gemma 4 12B (unified multimodal)"
 * record, "required kernel class"), so a bare streaming read with the decode kernels' own
 * loads (16 bytes per lane, non-temporal, one contiguous KiB per instruction, 16 in flight
 * per wave, four waves per CU) gives the rate no decode kernel can beat on this device.
 * gemma_stream_read reads `bytes` (a non-zero multiple of 1024) of device memory at src
 * (16-byte aligned) once, on `stream`, and writes a reduction of what it read to sink
 * (device, 16-byte aligned, gemma_stream_read_sink_bytes() bytes) so that nothing is
 * skipped.  Errors: GA_ERR_NULL, GA_ERR_DIMS, GA_ERR_ARCH, GA_ERR_LAUNCH.
 */
size_t gemma_stream_read_sink_bytes(void);
int32_t gemma_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Precondition flags written by gemma_attn_validate, per batch row. */
enum {
  GA_FLAG_QPOS_GE_CTX = 1, /* q_pos >= ctx                                         */
  GA_FLAG_EVICTED = 2,     /* ring: the window (or full attention) needs overwritten slots */
  GA_FLAG_LINEAR_OVER = 4, /* linear: ctx > C                                      */
  GA_FLAG_NEGATIVE = 8,    /* ctx < 0 or q_pos < 0                                 */
  GA_FLAG_OVER_MAX_CTX = 16 /* ctx > shape->max_ctx (the workspace bound)          */
};

/*
 * Debug check of the device-side preconditions: writes GA_FLAG_* bits for each row to
 * dev_flags (device int32 [B]) on `stream`.  The decode itself does not need it.  Host
 * arguments are checked as for the decode (same status codes, nothing launched on error).
 * Passage: "Gemma 4 12B (unified multimodal)" record, "(6) On Apple Silicon": a cache
 * class that silently grows past its bound or fails only on the first request; this call
 * reports at call time, per row, which device-side precondition a decode would violate
 * (the decode itself clamps every index and never reads out of bounds).
 */
int32_t gemma_attn_validate(const ga_shape* shape, const int32_t* ctx_lens, const int32_t* q_pos,
                            int32_t window, int32_t* dev_flags, void* stream);

/* gemma_attn_validate for T = num_tokens tokens per row at q_pos[b] + t: dev_flags is
 * device int32 [B, T]. */
int32_t gemma_attn_validate_multi(const ga_shape* shape, int32_t num_tokens,
                                  const int32_t* ctx_lens, const int32_t* q_pos, int32_t window,
                                  int32_t* dev_flags, void* stream);

/*
 * Debug dump of the key range each row attends to, computed by the same device code
 * the decode kernels use: dev_out (device int32 [B, 4]) receives
 * (lo, hi, slot(lo), n) with n = hi - lo + 1 (n = 0 and lo = hi + 1 for an empty row).
 * Passage: "Gemma 4 12B (unified multimodal)" record, "required kernel class" (a local
 * layer reads exactly w entries) and "(2) On B200" (a kernel that picked the wrong window
 * keys at some sequence-length alignments): the dump lets a caller check, bit for bit,
 * which positions the kernels select.  Errors as for gemma_attn_validate.
 */
int32_t gemma_attn_debug_ranges(const ga_shape* shape, const int32_t* ctx_lens,
                                const int32_t* q_pos, int32_t window, int32_t* dev_out,
                                void* stream);

/* Static description of a status code (never NULL).  Every failure is reported by a
 * distinct code at call time rather than silently ("Gemma 4 12B (unified multimodal)"
 * record, "(6) On Apple Silicon"). */
const char* gemma_attn_strerror(int32_t status);

/* Library version, as major * 10000 + minor * 100 + patch (no passage: bookkeeping). */
int32_t gemma_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA_ATTN_H */
