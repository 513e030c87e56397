/*
 * oracle.h -- plain fp64 CPU reference of one decode step of a Q4_0-weight
 * decoder (Qwen3 / Gemma-4 style).  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg call it; the product
 * library never does.  It shares no code, header or table with the HIP path.
 *
 * All floating-point arithmetic is fp64 and scalar, in the index order of the
 * definitions; the only narrowing is where the pages fix a storage type
 * (binary16 block scales, F32 KV-cache rows).
 *
 * Pages cited (by title and section):
 *   [GEM]  "Research record" (gem engine research record), sections
 *          "Verified model facts" and "Native Metal diagnostic: buffer
 *          ownership".
 *   [GELO] "GELO LLM" (generation), sections 02 "Definitions & glossary",
 *          04 "Supported workloads & architectures", 05 "Components",
 *          06 "Compute flow & trust boundaries".
 *
 * Parity status of each function is listed next to it: every function is
 * pinned by the CPU tests except orc_decode_step, whose whole-step result is
 * only pinned through its pinned parts ("parity unpinned" beyond that
 * composition: the pages print no worked decode example).
 */
#ifndef Q4DEC_ORACLE_H
#define Q4DEC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 -> fp64, exact ([GEM] Native Metal diagnostic: the Q4_0
 * scales are binary16).  Pinned: all 65,536 patterns vs a library conversion. */
double orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double v);  /* nearest binary16, ties to even */
void orc_geglu(const double *g, const double *u, int64_t n, double *h);
void orc_softcap(double *v, int64_t n, double c);

/* Dequantise an n_rows x k Q4_0 / Q8_0 matrix (row-major block rows) to fp64.
 * Pinned: hand-worked block, unit vectors, Q4_0 vs Q8_0 cross-encoding. */
void orc_q4_0_dequant(const uint8_t *w, int64_t n_rows, int64_t k, double *out);
void orc_q8_0_dequant(const uint8_t *w, int64_t n_rows, int64_t k, double *out);

/* y[b][n] = sum_k W[n][k] * x[b][k] (+ res[b][n]); terms[b][n] = sum_k |W x|
 * (+ |res|).  x is [B][K], y/res/terms are [B][N].  res/terms may be NULL.
 * Pinned: hand-worked block, linearity, integer-exact special case. */
void orc_q4_0_matvec(const uint8_t *w, int64_t n_rows, int64_t k, const double *x,
                     int64_t batch, const double *res, double *y, double *terms);
void orc_q8_0_matvec(const uint8_t *w, int64_t n_rows, int64_t k, const double *x,
                     int64_t batch, const double *res, double *y, double *terms);

/* x[b][:] = dequantised row tok[b] of a Q8_0 table (tied embedding).
 * Pinned: equals the unit-vector matvec of the same table. */
void orc_q8_0_gather(const uint8_t *table, int64_t vocab, int64_t k, const int32_t *tok,
                     int64_t batch, double *x);

/* y = w * x / sqrt(mean(x^2) + eps) per row; w == NULL means unit gain.
 * Pinned: unit-RMS invariant, constant-row closed form. */
void orc_rmsnorm(const double *x, const double *w, int64_t rows, int64_t dim, double eps,
                 double *y);

/* NeoX rotary embedding of one head vector of length hd, in place, at
 * position pos: pair (i, i + hd/2), angle pos * theta^(-2i/hd).
 * Pinned: identity at 0, norm preservation, relative-position property,
 * hand-computed pair rotation, NeoX (not interleaved) pairing. */
void orc_rope_neox(double *x, int64_t hd, int64_t pos, double theta);

/* h = g * u / (1 + exp(-g)).  Pinned: silu(0)=0, asymptotes, exact values. */
void orc_swiglu(const double *g, const double *u, int64_t n, double *h);

/* Index of the largest value, lowest index on ties; *margin = top1 - top2.
 * Pinned: brute force with crafted ties. */
int64_t orc_argmax(const double *v, int64_t n, double *margin);

/* Decode attention of one sequence with grouped-query heads.
 *   q      [n_q_heads][hd]
 *   keys   [n_pos][n_kv_heads][hd], values likewise, position-indexed 0..n_pos-1
 *   window 0 = all positions, else only positions >= n_pos - window are seen
 *   o      [n_q_heads][hd]
 *   bound  [n_q_heads][hd] (may be NULL): sum_j p_j |v_j| + sum_j p_j |v_j - o| S_j,
 *          S_j = scale * sum_i |q_i k_ji|  (first-order error-propagation weight)
 * Query head h reads kv head h / (n_q_heads / n_kv_heads).
 * Pinned: softmax weights sum to 1, single key, equal keys, window 1, MHA case,
 * head-group mapping, chunked-merge composition, small brute force. */
void orc_gqa_attention(const double *q, int64_t n_q_heads, int64_t n_kv_heads, int64_t hd,
                       const double *keys, const double *values, int64_t n_pos,
                       int64_t window, double scale, double *o, double *bound);

/* ------------------------------------------------------------------ decode step */
typedef struct {
    const uint8_t *wqkv;      /* Q4_0 [(Hq + Hkv + (v_from_k ? 0 : Hkv)) * hd][d_model] */
    const uint8_t *wo;        /* Q4_0 [d_model][Hq * hd] */
    const uint8_t *wgu;       /* Q4_0 [2 * ffn][d_model]: gate rows then up rows */
    const uint8_t *wd;        /* Q4_0 [d_model][ffn] */
    const double *attn_norm;  /* [d_model] */
    const double *ffn_norm;   /* [d_model] */
    const double *q_norm;     /* [hd] */
    const double *k_norm;     /* [hd] */
    void *k_cache;            /* [batch][Hkv][cap][hd], slot = position mod cap */
    void *v_cache;            /* fp32, or binary16 when kv_f16 */
    int64_t n_kv_heads, head_dim, cap, window;
    double rope_theta, attn_scale;
    int32_t v_from_k;         /* 1: no v rows; v = unit-gain rmsnorm of raw k */
    int32_t kv_f16;           /* 1: binary16 caches (rows appended rounded to nearest) */
    int64_t rope_dims;        /* rotated dims (p-RoPE); 0 = all of head_dim */
    const double *post_attn_norm; /* sandwich post-norm gains [d_model], or NULL */
    const double *post_ffn_norm;
} orc_layer;

typedef struct {
    int64_t n_layers, d_model, n_q_heads, ffn, vocab, batch;
    double eps;
    const uint8_t *embed;     /* Q8_0 [vocab][d_model], tied input/output table */
    const double *final_norm; /* [d_model] */
    orc_layer *layers;
    int32_t ffn_act;          /* 0: SwiGLU (SiLU gate); 1: GeGLU (tanh-form GELU gate) */
    double embed_scale;       /* gathered rows times this (0: unscaled) */
    double logit_softcap;     /* logits c tanh(l / c) (0: none) */
} orc_model;

/* One greedy decode step for all batch rows at position pos (rows of the new
 * token are written into the caches at slot pos % cap).  logits may be NULL
 * ([batch][vocab]); margins may be NULL ([batch]).  Parity unpinned beyond
 * the composition of pinned parts. */
void orc_decode_step(const orc_model *m, int64_t pos, const int32_t *tok, int32_t *next,
                     double *logits, double *margins);

int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
