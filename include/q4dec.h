/*
 * q4dec.h -- C ABI of the MI355X (gfx950) decode hot path for Q4_0-weight
 * decoders: Q4_0/Q8_0 dequant-matvec, embedding gather, RMSNorm, per-head
 * QK-norm + NeoX RoPE with KV-cache append, split-K grouped-query decode
 * attention, SwiGLU, greedy argmax, and a decode scheduler that replays one
 * whole decode step as a HIP graph.
 *
 * Pages cited (by title and section):
 *   [GEM]  "Research record" (gem engine research record): "Verified model
 *          facts"; "Native Metal diagnostic: buffer ownership".
 *   [GELO] "GELO LLM" (generation): 02 "Definitions & glossary", 04
 *          "Supported workloads & architectures", 05 "Components", 06
 *          "Compute flow & trust boundaries".
 *
 * Conventions for every call:
 *   - Pointers named *_dev or documented as device memory must point to
 *     device memory of the current HIP device; the caller owns all memory.
 *     The library never allocates, frees or keeps device memory of its own.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; nothing synchronises the
 *     device except decode_model_create.
 *   - Activations are fp32, row-major, batch-major ([B][dim]).
 *   - Arguments are validated on the host before any HIP call; a call that
 *     returns an error has enqueued nothing.  The message of the last error
 *     of the calling thread is returned by q4dec_last_error().
 *   - Q4_0 / Q8_0 matrices are row-major block rows: row n (output feature n)
 *     holds K/32 consecutive blocks.
 */
#ifndef Q4DEC_H
#define Q4DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q4_OK = 0,
    Q4_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad flag */
    Q4_ERR_SHAPE = 2,       /* sizes inconsistent (K % 32, Hq % Hkv, odd head_dim, ...) */
    Q4_ERR_ALIGNMENT = 3,   /* pointer not aligned as the call requires */
    Q4_ERR_CAPACITY = 4,    /* a position does not fit the KV cache */
    Q4_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    Q4_ERR_UNSUPPORTED = 6, /* valid but outside what the kernels implement */
    Q4_ERR_HIP = 7          /* the HIP runtime reported an error */
} q4_status;

/* Message of the calling thread's most recent error ("" if none). */
const char *q4dec_last_error(void);
/* Library version string. */
const char *q4dec_version(void);

/* ------------------------------------------------------------------ matvec
 * q4_0_matvec: y[b][n] = sum_k W[n][k] * x[b][k]  (+ residual[b][n])
 *   with W[n][k] = d * (q - 8) for the Q4_0 block holding element k of row n:
 *   18 bytes = little-endian binary16 scale d, then 16 code bytes; byte j
 *   holds element j (low nibble) and element j + 16 (high nibble).
 *   ([GEM] Native Metal diagnostic: 18-byte blocks, binary16 scale, 16
 *   payload bytes, (quant - 8) * scale.)
 *
 *   W         device, N * (K/32) * 18 bytes, 2-byte aligned
 *   N, K      output / input features; K % 32 == 0; N >= 1; 1 <= B <= 8
 *   x         device fp32 [B][K], 4-byte aligned
 *   y         device fp32 [B][N]; may alias residual (in-place residual add)
 *   residual  device fp32 [B][N] or NULL
 * Accumulation is fp32; every weight-activation product is formed exactly
 * (on the matrix cores: activations as two binary16 halves with a power-of-two
 * scale per 256 elements, about 22 significant bits).
 * B > 1 without a workspace: from B = 3, when K % 256 == 0, W and x are
 * 16-byte aligned, y does not overlap x and the matrix has many rows
 * (N >= 16384, or N >= 4096 at B >= 6), the matrix-core tile kernel with every
 * workgroup walking the whole K reads W once per call; otherwise the B = 1
 * vector kernel runs once per activation row (the rows side by side in one
 * launch) and W is read B times, from HBM or from the last-level cache.  The
 * matrix-core entry q4_0_matvec_batched, which splits K and takes a
 * workspace, is faster on most shapes from B = 2 on.
 * Errors: Q4_ERR_INVALID_ARG (null / sizes), Q4_ERR_SHAPE (K % 32),
 *         Q4_ERR_ALIGNMENT, Q4_ERR_UNSUPPORTED (B > 8), Q4_ERR_HIP.
 */
q4_status q4_0_matvec(const void *W, int64_t N, int64_t K, const float *x, int64_t B,
                      float *y, const float *residual, void *stream);

/* q8_0_matvec: as q4_0_matvec for Q8_0 blocks: 34 bytes = little-endian
 * binary16 scale d then 32 int8 codes q; W[n][k] = d * q.  Used for the tied
 * logit projection ([GEM] Verified model facts: Q8_0 token table; [GELO] 04:
 * tied input/output embeddings).  Same arguments and errors. */
q4_status q8_0_matvec(const void *W, int64_t N, int64_t K, const float *x, int64_t B,
                      float *y, const float *residual, void *stream);

/* Input transforms a matvec can apply to its activation rows as it reads
 * them, fusing the producer of the input into the matvec:
 *   Q4_IN_PLAIN    x
 *   Q4_IN_RMSNORM  norm_w * x / sqrt(mean(x^2) + eps)  (norm_w NULL: unit gain)
 *                  ([GELO] 05 Components: decoder RMSNorm)
 *   Q4_IN_SWIGLU   x / (1 + exp(-x)) * x2               ([GELO] 04: SwiGLU FFN)
 *   Q4_IN_GEGLU    gelu(x) * x2, gelu in its tanh form  ([GELO] generation page, Gemma 4
 *                  blockers: gelu_pytorch_tanh): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
typedef enum { Q4_IN_PLAIN = 0, Q4_IN_RMSNORM = 1, Q4_IN_SWIGLU = 2, Q4_IN_GEGLU = 3 } q4_input_op;

/* Output transforms:
 *   Q4_OUT_PLAIN   y[b][n] = z[b][n] (+ residual[b][n]),  z = W op(x), y [B][N]
 *   Q4_OUT_SWIGLU  y[b][p] = z[b][p] / (1 + exp(-z[b][p])) * z[b][p + N/2]
 *                  for p < N/2, y [B][N/2]: a merged gate|up projection that
 *                  hands the FFN activation straight to the down projection
 *                  ([GELO] 04: SwiGLU FFN; 06: merged gate|up); N even, no
 *                  residual.
 *   Q4_OUT_GEGLU   the same with gelu (tanh form) in place of x / (1 + exp(-x)). */
typedef enum { Q4_OUT_PLAIN = 0, Q4_OUT_SWIGLU = 1, Q4_OUT_GEGLU = 2 } q4_output_op;

/* q4_0_matvec_fused / q8_0_matvec_fused: y[b] = out_op(W op(x[b])) (+ residual[b]),
 * where row b of x (and of x2 for SwiGLU) starts at element b * ld_x
 * (ld_x >= K; a merged gate|up output passes x = gu, x2 = gu + F, ld_x = 2F).
 * The transform is computed in fp32 exactly as rmsnorm() / swiglu() define
 * it (the RMSNorm sum of squares may be added in a different order).
 * Other arguments, layouts and errors as q4_0_matvec / q8_0_matvec, plus
 * Q4_ERR_INVALID_ARG for an unknown op or out_op, a missing x2, eps < 0, or
 * a SwiGLU output with odd N or a residual; Q4_ERR_SHAPE for ld_x < K; and
 * Q4_ERR_UNSUPPORTED for a SwiGLU output unless K % 256 == 0, K <= 8192 and
 * x, x2, norm_w are 16-byte aligned with ld_x % 4 == 0. */
q4_status q4_0_matvec_fused(const void *W, int64_t N, int64_t K, const float *x, const float *x2,
                            int64_t ld_x, int64_t B, q4_input_op op, q4_output_op out_op,
                            const float *norm_w, float eps, float *y, const float *residual,
                            void *stream);
q4_status q8_0_matvec_fused(const void *W, int64_t N, int64_t K, const float *x, const float *x2,
                            int64_t ld_x, int64_t B, q4_input_op op, q4_output_op out_op,
                            const float *norm_w, float eps, float *y, const float *residual,
                            void *stream);

/* q4_0_matvec_post_norm: a sandwich-norm block boundary and the next
 * projection in one call ([GEM] 31B trace: post-sublayer RMSNorm, residual
 * add, then the next pre-norm RMSNorm and projection):
 *   h_out[b] = h[b] + post_w * z[b] / sqrt(mean(z[b]^2) + eps)
 *   y[b]     = out_op(W (pre_w * h_out[b] / sqrt(mean(h_out[b]^2) + eps)))
 * (pre_w NULL: unit gain).  Rows b of h, z and h_out start at b * ld; y is
 * [B][N] ([B][N/2] for a gated out_op).  B <= 8 (vector units); every
 * workgroup computes h_out itself and one per row writes it, so h_out must
 * not overlap h or z.
 *   W       16-bit aligned Q4_0 [N][K/32] blocks; K % 256 == 0, K <= 8192
 *   h, z, h_out, post_w, pre_w   16-byte aligned, ld % 4 == 0, ld >= K
 *   y       must not overlap h, z or h_out
 * Errors: Q4_ERR_INVALID_ARG (NULL, sizes, eps < 0, odd N with a gated output,
 * overlap), Q4_ERR_SHAPE (ld < K), Q4_ERR_ALIGNMENT, Q4_ERR_UNSUPPORTED (B > 8,
 * K), Q4_ERR_HIP. */
q4_status q4_0_matvec_post_norm(const void *W, int64_t N, int64_t K, const float *h,
                                const float *z, int64_t ld, int64_t B, const float *post_w,
                                const float *pre_w, float eps, float *h_out,
                                q4_output_op out_op, float *y, void *stream);

/* q4_0_matvec_batched / q8_0_matvec_batched: the same products as the fused
 * calls, computed on the matrix cores for 1 <= B <= 32 activation rows; meant
 * for B >= 2, where eight products per weight outrun the vector units.  Rows
 * are taken in groups of 8; the groups of one row range run back to back on
 * one XCD, so the weights are read from HBM once per call.
 * Operands are exact binary16 (codes as integers; activations, after a
 * power-of-two scaling per row and per 256 k, split into two halves), so
 * every product is exact and sums are fp32.  RMSNorm's 1/rms is applied to
 * the finished sums.  One kernel launch; bitwise reproducible.
 *   W         16-byte aligned; K % 256 == 0 (else Q4_ERR_UNSUPPORTED)
 *   x, x2     16-byte aligned, ld_x % 4 == 0; norm_w 16-byte aligned
 *   y         must not overlap x or x2 (Q4_ERR_INVALID_ARG); may alias residual;
 *             a SwiGLU output (out_op) is supported for every K % 256 == 0
 *   ws        device workspace of at least matvec_batched_workspace(N, K, B)
 *             bytes, 256-byte aligned, owned by the caller.  Its first 512 KiB
 *             (split tickets) must be zero before the first call that uses
 *             it; every call leaves them zero.  Calls sharing a workspace
 *             must be ordered (one stream).
 * Other arguments and errors as q4_0_matvec_fused, plus Q4_ERR_WORKSPACE. */
size_t matvec_batched_workspace(int64_t N, int64_t K, int64_t B);
q4_status q4_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                              const float *x2, int64_t ld_x, int64_t B, q4_input_op op,
                              q4_output_op out_op, const float *norm_w, float eps, float *y,
                              const float *residual, void *ws, size_t ws_bytes, void *stream);
q4_status q8_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                              const float *x2, int64_t ld_x, int64_t B, q4_input_op op,
                              q4_output_op out_op, const float *norm_w, float eps, float *y,
                              const float *residual, void *ws, size_t ws_bytes, void *stream);

/* q4_0_matvec_batched_noalloc: q4_0_matvec_batched without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments (less ws / ws_bytes), results bit-identical to
 * q4_0_matvec_batched's, same errors.  The split tickets, sums of squares and
 * split-K partials live in a static device array of
 * Q4_NOALLOC_SCRATCH_BYTES per device, held until the process ends; a shape
 * whose plan needs more (matvec_batched_workspace(N, K, B) > that size)
 * returns Q4_ERR_UNSUPPORTED before any HIP call.  The call allocates and
 * frees nothing.  The first call on a device looks the array up and clears
 * its tickets with a small kernel on `stream`; every call leaves them zero.
 * All calls on one device share the array: calls that overlap in time (on
 * different streams, or from several threads without ordering) race and
 * give undefined results. */
#define Q4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
q4_status q4_0_matvec_batched_noalloc(const void *W, int64_t N, int64_t K, const float *x,
                                      const float *x2, int64_t ld_x, int64_t B, q4_input_op op,
                                      q4_output_op out_op, const float *norm_w, float eps,
                                      float *y, const float *residual, void *stream);

/* q8_0_gather: x[b][:] = dequantised row tokens[b] of the Q8_0 table E
 * (embedding lookup of the tied table; [GELO] 05 generation loop embeds the
 * previous token).
 *   E       device, V * (K/32) * 34 bytes;  tokens device int32 [B]
 *   x       device fp32 [B][K]
 * A token id outside [0, V) yields a row of NaN (no out-of-range read).
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_SHAPE (K % 32), Q4_ERR_HIP. */
q4_status q8_0_gather(const void *E, int64_t V, int64_t K, const int32_t *tokens, int64_t B,
                      float *x, void *stream);

/* q8_0_gather_scaled: the same rows times scale (Gemma-4 multiplies the
 * embedding by sqrt(d_model); the value is the caller's).  x = (d * q) * scale
 * per element.  Errors as q8_0_gather. */
q4_status q8_0_gather_scaled(const void *E, int64_t V, int64_t K, const int32_t *tokens,
                             int64_t B, float scale, float *x, void *stream);

/* ------------------------------------------------------------------ norms
 * rmsnorm: y[r][i] = w[i] * x[r][i] / sqrt(mean_i(x[r][i]^2) + eps)
 *   ([GELO] 05 Components: decoder RMSNorm.)  x, y device fp32 [rows][dim]
 *   (y may alias x); w device fp32 [dim] or NULL for unit gain; eps >= 0.
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_HIP. */
q4_status rmsnorm(const float *x, const float *w, int64_t rows, int64_t dim, float eps,
                  float *y, void *stream);

/* rmsnorm_add: x[r][i] += w[i] * y[r][i] / sqrt(mean_i(y[r][i]^2) + eps), the
 *   post-sublayer RMSNorm of a sandwich-norm block joining the residual
 *   stream x ([GEM] 31B trace: post-attention RMSNorm, residual add, FFN
 *   RMSNorm).  y, x device fp32 [rows][dim], not overlapping; w [dim] or NULL.
 * Errors: Q4_ERR_INVALID_ARG (NULL, sizes, overlap), Q4_ERR_ALIGNMENT, Q4_ERR_HIP. */
q4_status rmsnorm_add(const float *y, const float *w, int64_t rows, int64_t dim, float eps,
                      float *x, void *stream);

/* swiglu: h[r][i] = g[r][i] / (1 + exp(-g[r][i])) * u[r][i], 0 <= i < n.
 *   ([GELO] 04: SwiGLU FFN.)  g and u are read with row stride ld (ld >= n;
 *   a merged gate|up projection output passes g = gu, u = gu + n, ld = 2n);
 *   h is [rows][n].  Device fp32.
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_HIP. */
q4_status swiglu(const float *g, const float *u, int64_t rows, int64_t n, int64_t ld, float *h,
                 void *stream);

/* geglu: as swiglu with gelu (tanh form) in place of SiLU:
 *   h = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u
 *   ([GELO] generation page, Gemma 4 blockers: gelu_pytorch_tanh). */
q4_status geglu(const float *g, const float *u, int64_t rows, int64_t n, int64_t ld, float *h,
                void *stream);

/* softcap: v[i] = cap * tanh(v[i] / cap) in place, cap > 0 (final-logit soft
 *   capping; [GELO] generation page, Gemma 4: final_logit_softcapping).  The
 *   map is increasing, so the greedy choice is unchanged.  v device fp32 [n].
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_ALIGNMENT, Q4_ERR_HIP. */
q4_status softcap(float *v, int64_t n, float cap, void *stream);

/* KV-cache layout: element strides of a [batch][n_kv_heads][cap][head_dim]
 * style cache; the head_dim axis is contiguous.  Position p of a sequence
 * lives in slot p % cap (a cache with cap >= the positions it must hold is
 * linear; a sliding-window layer may use a ring with cap == window).
 * dtype: the cache elements, fp32 or binary16.  A binary16 cache halves the
 * attention bytes; appended rows are computed in fp32 and rounded to the
 * nearest binary16 (ties to even), and cached elements are read exactly. */
typedef enum { Q4_KV_F32 = 0, Q4_KV_F16 = 1 } q4_kv_dtype;
typedef struct {
    int64_t batch, n_kv_heads, head_dim, cap;
    int64_t stride_b, stride_h, stride_t;
    int64_t dtype; /* q4_kv_dtype */
} q4_kv_layout;

/* qk_norm_rope: for the new token of each sequence b at device position
 * *pos_dev:
 *   q_h <- RoPE(rmsnorm(q_h, q_norm))  for each query head (in place in q);
 *   k_g <- RoPE(rmsnorm(k_g, k_norm)), appended to k_cache at slot pos % cap;
 *   v_g appended to v_cache; with v_from_k the V row is the unit-gain
 *   rmsnorm of the raw (pre-norm) k_g and v must be NULL.
 * RoPE is NeoX style: element i pairs with i + hd/2, angle
 * pos * theta^(-2i/hd), computed in fp64 and reduced before the sine/cosine.
 * ([GELO] 02 glossary and 05 Components: per-head QK-norm before RoPE with a
 * shared head_dim gain; [GEM] Native Metal diagnostic: NeoX RoPE; [GEM]
 * Verified model facts: full-attention layers take V from the K projection
 * with an unweighted RMS normalisation.)
 *   q        device fp32, row b at q + b*ldq, n_q_heads * head_dim values
 *   k, v     device fp32, row b at k + b*ldkv (same for v)
 *   q_norm, k_norm  device fp32 [head_dim]
 *   kv       cache layout (host struct); head_dim even, <= 512
 *   k_cache, v_cache  device, elements of kv->dtype
 *   pos_dev  device int64 [1]; the kernel writes nothing outside the cache
 *            (a position whose slot would be out of range is not written).
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_SHAPE (n_q_heads % n_kv_heads, odd hd),
 *         Q4_ERR_UNSUPPORTED (hd > 512), Q4_ERR_HIP. */
q4_status qk_norm_rope(float *q, int64_t ldq, const float *k, const float *v, int64_t ldkv,
                       const float *q_norm, const float *k_norm, int64_t n_q_heads,
                       const q4_kv_layout *kv, const int64_t *pos_dev, double theta,
                       float eps, int v_from_k, void *k_cache, void *v_cache,
                       void *stream);

/* qk_norm_rope_partial: qk_norm_rope with p-RoPE ([GELO] generation page,
 * glossary: only the first p * head_dim dimensions rotate, the rest pass
 * through; Gemma 4 global layers use p = 0.25).  Reading: elements
 * [0, rot_dims) rotate as a NeoX rotation of a rot_dims-dimensional vector
 * (pairs i, i + rot_dims/2, angle pos * theta^(-2i/rot_dims)); elements
 * [rot_dims, head_dim) are normalised only.  rot_dims even, 2..head_dim
 * (head_dim: qk_norm_rope).  Errors as qk_norm_rope. */
q4_status qk_norm_rope_partial(float *q, int64_t ldq, const float *k, const float *v,
                               int64_t ldkv, const float *q_norm, const float *k_norm,
                               int64_t n_q_heads, const q4_kv_layout *kv, const int64_t *pos_dev,
                               double theta, float eps, int v_from_k, int64_t rot_dims,
                               void *k_cache, void *v_cache, void *stream);

/* ------------------------------------------------------------------ attention
 * gqa_decode_attn: one query row per sequence attends the cached positions
 *   [lo, n) with n = *n_dev and lo = max(0, n - window) (window 0 = all):
 *   out_h = sum_j softmax_j(scale * q_h . k_j) v_j, query head h reading kv
 *   head h / (n_q_heads / n_kv_heads).
 *   ([GELO] 05: cached GQA attention, decode attends n_cache + 1 keys; 02:
 *   GQA, sliding window over the last W tokens.)
 * Split-K: the key range is cut into fixed chunks processed in parallel, each
 * producing (max, sum, weighted V); a second pass merges the chunks in
 * ascending order, so results are bitwise reproducible.
 *   q        device fp32, row b at q + b*ldq ([n_q_heads][head_dim])
 *   k_cache, v_cache  device, elements of kv->dtype, with layout kv
 *            (slot = position % cap); 16-byte aligned, strides multiples of 4
 *   n_dev    device int64 [1]; positions outside the last cap are never read
 *   out      device fp32, row b at out + b*ldo ([n_q_heads][head_dim])
 *   ws       device workspace of at least gqa_decode_attn_workspace() bytes,
 *            256-byte aligned; contents need no initialisation
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_SHAPE, Q4_ERR_UNSUPPORTED (hd > 512 or
 *         hd % 4, group > 16), Q4_ERR_WORKSPACE, Q4_ERR_HIP. */
q4_status gqa_decode_attn(const float *q, int64_t ldq, int64_t n_q_heads, const void *k_cache,
                          const void *v_cache, const q4_kv_layout *kv, const int64_t *n_dev,
                          int64_t window, float scale, float *out, int64_t ldo, void *ws,
                          size_t ws_bytes, void *stream);

/* Workspace bytes gqa_decode_attn needs for this layout / window (0 on bad
 * arguments). */
size_t gqa_decode_attn_workspace(const q4_kv_layout *kv, int64_t n_q_heads, int64_t window);

/* gqa_decode_attn_rope: qk_norm_rope followed by gqa_decode_attn in one call,
 * reading q, k (and v) raw from the merged projection row: per head
 * RMSNorm with q_norm / k_norm, NeoX RoPE at the position *pos_dev, the new
 * key and value rows appended at slot pos % cap (v = unit-gain RMSNorm of the
 * raw key when v_from_k), then attention over the n = pos + 1 positions as
 * gqa_decode_attn.  The normalised q is not written back.
 * ([GELO] 05 Components: cached GQA attention with per-head QK-norm before
 * RoPE; [GEM] Verified model facts: V from K on full-attention layers.)
 *   qkv      device fp32 [B][ld]: q (n_q_heads * hd) | k (Hkv * hd) | v (Hkv * hd,
 *            absent when v_from_k); 16-byte aligned, ld % 4 == 0
 *   pos_dev  device int64: the position of the new token
 * Other arguments, the workspace and errors as qk_norm_rope / gqa_decode_attn. */
q4_status gqa_decode_attn_rope(const float *qkv, int64_t ld, int64_t n_q_heads,
                               const float *q_norm, const float *k_norm, const q4_kv_layout *kv,
                               const int64_t *pos_dev, double theta, float eps, int v_from_k,
                               void *k_cache, void *v_cache, int64_t window, float scale,
                               float *out, int64_t ldo, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ sampling
 * argmax_rows: out[b] = index of the largest logits[b][v], lowest index on
 *   ties ([GELO] 05: greedy sampler; [GEM] Native Metal diagnostic: equal
 *   logits resolve deterministically by token id).  NaN never wins.
 *   logits device fp32 [B][V]; out device int32 [B].
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_HIP. */
q4_status argmax_rows(const float *logits, int64_t B, int64_t V, int32_t *out, void *stream);

/* argmax_rows_ws: the same choice in two passes with a caller-owned device
 * workspace of argmax_rows_workspace(B) bytes (4-byte aligned, no
 * initialisation needed): 64 workgroups per row reduce slices, then one
 * wavefront per row reduces the slices in order.  Calls sharing a workspace
 * must be ordered.  Errors as argmax_rows, plus Q4_ERR_WORKSPACE. */
size_t argmax_rows_workspace(int64_t B);
q4_status argmax_rows_ws(const float *logits, int64_t B, int64_t V, int32_t *out, void *ws,
                         size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ decode step
 * One autoregressive decode step of a pre-norm decoder ([GELO] 06 Compute
 * flow: per block RMSNorm -> merged QKV projection -> per-head QK-norm +
 * RoPE -> cached GQA attention -> O projection + residual -> RMSNorm ->
 * merged gate|up -> SwiGLU -> down projection + residual; tied Q8_0 logits;
 * greedy choice), with the whole step captured once and replayed as a HIP
 * graph ([GEM] Native Metal diagnostic: persistent buffers and whole-token
 * command spans).  All weights and caches stay resident; the position lives
 * in device memory so the same graph serves every step. */
typedef struct {
    const void *wqkv;        /* Q4_0 [(Hq + Hkv + (v_from_k ? 0 : Hkv)) * hd][d_model] */
    const void *wo;          /* Q4_0 [d_model][Hq * hd] */
    const void *wgu;         /* Q4_0 [2 * ffn][d_model]: gate rows, then up rows */
    const void *wd;          /* Q4_0 [d_model][ffn] */
    const float *attn_norm;  /* [d_model] */
    const float *ffn_norm;   /* [d_model] */
    const float *q_norm;     /* [hd] */
    const float *k_norm;     /* [hd] */
    void *k_cache;           /* [batch][Hkv][cap][hd], contiguous, elements of kv_dtype */
    void *v_cache;           /* same layout */
    int64_t n_kv_heads, head_dim, cap, window; /* window 0 = full attention */
    double rope_theta;
    float attn_scale;
    int32_t v_from_k;        /* 1: no V rows in wqkv; V = unit-gain rmsnorm(raw K) */
    int32_t kv_dtype;        /* q4_kv_dtype of both caches */
    /* Gemma-4 block variants (zero / NULL: the plain pre-norm block) */
    int64_t rope_dims;       /* rotated dims (p-RoPE, qk_norm_rope_partial); 0 = head_dim */
    const float *post_attn_norm; /* [d_model]: sandwich post-norm of the attention output */
    const float *post_ffn_norm;  /* [d_model]: sandwich post-norm of the FFN output */
} q4_layer_desc;

typedef struct {
    /* batch 1..8; up to 32 when every projection runs on the matrix cores
     * (d_model, ffn and n_q_heads * head_dim multiples of 256, weights
     * 16-byte aligned), else Q4_ERR_UNSUPPORTED */
    int64_t n_layers, d_model, n_q_heads, ffn, vocab, batch;
    float eps;
    const void *embed;        /* Q8_0 [vocab][d_model], tied input/output table */
    const float *final_norm;  /* [d_model] */
    const q4_layer_desc *layers; /* host array [n_layers], copied at create */
    /* Gemma-4 block variants (zero: off) */
    int32_t ffn_act;          /* 0: SwiGLU; 1: GeGLU (tanh-form GELU gate) */
    float embed_scale;        /* embedding rows times this (Gemma: sqrt(d_model)); 0 = 1 */
    float logit_softcap;      /* logits cap * tanh(l / cap); 0 = none */
} q4_model_desc;

typedef struct q4_decode_model q4_decode_model;

/* Device workspace bytes decode_model_create needs (activations, attention
 * partials, position counter). */
q4_status decode_model_workspace(const q4_model_desc *desc, size_t *bytes);

/* Validates the description, binds the caller's workspace (256-byte aligned,
 * at least decode_model_workspace() bytes) and returns a host handle.  The
 * position starts at 0.  Synchronises the device.
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_SHAPE, Q4_ERR_ALIGNMENT,
 *         Q4_ERR_UNSUPPORTED, Q4_ERR_WORKSPACE, Q4_ERR_HIP. */
q4_status decode_model_create(const q4_model_desc *desc, void *ws, size_t ws_bytes,
                              q4_decode_model **out);

/* Sets the position of the next token (all sequences advance in lockstep).
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_CAPACITY (pos does not fit a linear
 * cache), Q4_ERR_HIP. */
q4_status decode_model_set_position(q4_decode_model *m, int64_t pos, void *stream);

/* Current host-side view of the position of the next token. */
int64_t decode_model_position(const q4_decode_model *m);

/* Runs one step: tokens_dev (device int32 [batch]) are the current tokens;
 * writes the greedy next tokens to next_tokens_dev (device int32 [batch],
 * may equal tokens_dev) and, if logits_dev is not NULL, the logits (device
 * fp32 [batch][vocab]); then advances the position by one.  The first call
 * with a given (tokens, next, logits) pointer triple captures the graph;
 * later calls replay it.
 * Errors: Q4_ERR_INVALID_ARG, Q4_ERR_CAPACITY, Q4_ERR_HIP. */
q4_status decode_step(q4_decode_model *m, const int32_t *tokens_dev, int32_t *next_tokens_dev,
                      float *logits_dev, void *stream);

/* Same step, launched kernel by kernel instead of through the graph (for
 * debugging and for comparing the two).  Same arguments and errors. */
q4_status decode_step_eager(q4_decode_model *m, const int32_t *tokens_dev,
                            int32_t *next_tokens_dev, float *logits_dev, void *stream);

/* Releases the host handle and its graphs (caller memory is untouched). */
q4_status decode_model_destroy(q4_decode_model *m);

#ifdef __cplusplus
}
#endif
#endif /* Q4DEC_H */
