/*
 * oracle.c -- plain fp64 CPU reference for the decode hot path.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 * Independent of the HIP library: no shared code, headers or tables.
 *
 * Each function states the definition it writes out and where the pages give
 * it; the readings taken where the pages are silent are stated in place.
 * Loops run in the index order of the definition; OpenMP only splits
 * independent outputs (rows, heads), never a sum.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of later parallel regions started from the calling thread
 * (n >= 1; ignored otherwise).  Results do not depend on it: threads only
 * split independent outputs. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal: (1 + f/1024) * 2^(e-15); subnormal (e = 0): f * 2^-24.
 * [GEM] Native Metal diagnostic: block scales are binary16. */
double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)f, e - 25);
    return sign ? -v : v;
}

/* The binary16 nearest to v, ties to the even fraction (IEEE 754
 * roundTiesToEven): scale |v| to units of its binade's quantum (2^-24 for
 * subnormals, 2^(E-10) for 2^E <= |v| < 2^(E+1)), round to an integer with
 * rint (the default rounding mode is to nearest even), and carry a rounding
 * up to 2048 units into the next binade.  Magnitudes from 65520 up round to
 * infinity (65504 is the largest finite value; 65520 is the midpoint). */
uint16_t orc_double_to_half(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) {                 /* subnormal binade (or zero) */
        double u = rint(ldexp(a, 24));           /* 0 .. 1024; 1024 is the smallest normal */
        return (uint16_t)(sign | (uint16_t)u);
    }
    int e;
    (void)frexp(a, &e);                          /* a = m 2^e, m in [0.5, 1): E = e - 1 */
    int E = e - 1;
    double u = rint(ldexp(a, 10 - E));           /* 1024 .. 2048 */
    if (u == 2048.0) {
        u = 1024.0;
        E += 1;
    }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(u - 1024.0));
}

static double read_scale(const uint8_t *p) {
    /* little-endian byte order (the GGUF blocks are stored little-endian) */
    return orc_half_to_double((uint16_t)(p[0] | (p[1] << 8)));
}

/* Q4_0 block of 32 weights, 18 bytes ([GEM] Native Metal diagnostic: 18-byte
 * blocks, binary16 scale plus 16 payload bytes, weight = (quant - 8) * scale).
 * Code order inside the payload (the pages do not print it; reading taken
 * from the workload statement): byte j holds element j in its low nibble and
 * element j + 16 in its high nibble. */
static void q4_0_block(const uint8_t *blk, double *w32) {
    double d = read_scale(blk);
    const uint8_t *qs = blk + 2;
    for (int j = 0; j < 16; ++j) {
        int lo = qs[j] & 0x0F;
        int hi = qs[j] >> 4;
        w32[j] = d * (double)(lo - 8);
        w32[j + 16] = d * (double)(hi - 8);
    }
}

/* Q8_0 block of 32 weights, 34 bytes: binary16 scale then 32 int8 codes,
 * weight = code * scale ([GEM] Verified model facts: the token table is Q8_0;
 * the byte layout is the reading used throughout). */
static void q8_0_block(const uint8_t *blk, double *w32) {
    double d = read_scale(blk);
    for (int j = 0; j < 32; ++j)
        w32[j] = d * (double)(int8_t)blk[2 + j];
}

typedef void (*block_fn)(const uint8_t *, double *);

static void dequant_rows(block_fn fn, int block_bytes, const uint8_t *w, int64_t n_rows,
                         int64_t k, double *out) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_rows; ++n)
        for (int64_t b = 0; b < nb; ++b)
            fn(w + (n * nb + b) * block_bytes, out + n * k + b * 32);
}

void orc_q4_0_dequant(const uint8_t *w, int64_t n_rows, int64_t k, double *out) {
    dequant_rows(q4_0_block, 18, w, n_rows, k, out);
}

void orc_q8_0_dequant(const uint8_t *w, int64_t n_rows, int64_t k, double *out) {
    dequant_rows(q8_0_block, 34, w, n_rows, k, out);
}

/* y[b][n] = sum_k W[n][k] x[b][k] (+ res[b][n]), sum in increasing k. */
static void matvec(block_fn fn, int block_bytes, const uint8_t *w, int64_t n_rows, int64_t k,
                   const double *x, int64_t batch, const double *res, double *y,
                   double *terms) {
    int64_t nb = k / 32;
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < n_rows; ++n) {
            for (int64_t b = 0; b < nb; ++b)
                fn(w + (n * nb + b) * block_bytes, row + b * 32);
            for (int64_t bi = 0; bi < batch; ++bi) {
                const double *xb = x + bi * k;
                double s = 0.0, a = 0.0;
                for (int64_t i = 0; i < k; ++i) {
                    double t = row[i] * xb[i];
                    s += t;
                    a += fabs(t);
                }
                if (res) {
                    s += res[bi * n_rows + n];
                    a += fabs(res[bi * n_rows + n]);
                }
                y[bi * n_rows + n] = s;
                if (terms)
                    terms[bi * n_rows + n] = a;
            }
        }
        free(row);
    }
}

void orc_q4_0_matvec(const uint8_t *w, int64_t n_rows, int64_t k, const double *x,
                     int64_t batch, const double *res, double *y, double *terms) {
    matvec(q4_0_block, 18, w, n_rows, k, x, batch, res, y, terms);
}

void orc_q8_0_matvec(const uint8_t *w, int64_t n_rows, int64_t k, const double *x,
                     int64_t batch, const double *res, double *y, double *terms) {
    matvec(q8_0_block, 34, w, n_rows, k, x, batch, res, y, terms);
}

/* Embedding lookup of the tied Q8_0 table ([GELO] 04: tied input/output
 * embeddings; [GEM] Verified model facts: Q8_0 token embeddings). */
void orc_q8_0_gather(const uint8_t *table, int64_t vocab, int64_t k, const int32_t *tok,
                     int64_t batch, double *x) {
    int64_t nb = k / 32;
    (void)vocab;
    for (int64_t bi = 0; bi < batch; ++bi)
        for (int64_t b = 0; b < nb; ++b)
            q8_0_block(table + ((int64_t)tok[bi] * nb + b) * 34, x + bi * k + b * 32);
}

/* RMSNorm ([GELO] 05 Components: decoder rms_norm; 02 glossary: QK-norm is
 * the same per-head RMSNorm): y_i = w_i * x_i / sqrt((1/D) sum x^2 + eps).
 * Reading: the gain is w itself (not 1 + w). */
void orc_rmsnorm(const double *x, const double *w, int64_t rows, int64_t dim, double eps,
                 double *y) {
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * dim;
        double ss = 0.0;
        for (int64_t i = 0; i < dim; ++i)
            ss += xr[i] * xr[i];
        double inv = 1.0 / sqrt(ss / (double)dim + eps);
        for (int64_t i = 0; i < dim; ++i)
            y[r * dim + i] = xr[i] * inv * (w ? w[i] : 1.0);
    }
}

/* NeoX rotary embedding ([GEM] Native Metal diagnostic: NeoX RoPE): element
 * i is paired with element i + hd/2 and rotated by pos * theta^(-2i/hd). */
void orc_rope_neox(double *x, int64_t hd, int64_t pos, double theta) {
    int64_t half = hd / 2;
    for (int64_t i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -(2.0 * (double)i) / (double)hd);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = b * c + a * s;
    }
}

/* SwiGLU ([GELO] 04: SwiGLU FFN): h = silu(g) * u, silu(z) = z / (1 + e^-z). */
void orc_swiglu(const double *g, const double *u, int64_t n, double *h) {
    for (int64_t i = 0; i < n; ++i)
        h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* GeGLU with the tanh form of GELU ([GELO] generation page, Gemma 4
 * blockers: the FFN activation is gelu_pytorch_tanh rather than SiLU; the
 * tanh form is Hendrycks and Gimpel's approximation):
 * h = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u. */
void orc_geglu(const double *g, const double *u, int64_t n, double *h) {
    const double k = sqrt(2.0 / 3.14159265358979323846);
    for (int64_t i = 0; i < n; ++i) {
        double z = g[i];
        h[i] = 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z))) * u[i];
    }
}

/* Final-logit soft capping ([GELO] generation page, Gemma 4 developed list:
 * final_logit_softcapping wired through the logits): l <- c tanh(l / c). */
void orc_softcap(double *v, int64_t n, double c) {
    for (int64_t i = 0; i < n; ++i)
        v[i] = c * tanh(v[i] / c);
}

/* Greedy choice ([GELO] 05: greedy sampler; [GEM] Native Metal diagnostic:
 * equal logits resolve deterministically by token id -> lowest id wins). */
int64_t orc_argmax(const double *v, int64_t n, double *margin) {
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > v[best])
            best = i;
    if (margin) {
        double second = -INFINITY;
        for (int64_t i = 0; i < n; ++i)
            if (i != best && v[i] > second)
                second = v[i];
        *margin = n > 1 ? v[best] - second : INFINITY;
    }
    return best;
}

/* Decode attention ([GELO] 05: causal_gqa_attention_cached with one query
 * row attending every cached position plus the new one; 02 glossary: GQA
 * shares one K/V head among several query heads; sliding-window layers see
 * only the last W tokens).  Readings: head h reads kv head floor(h / G);
 * the window counts the current token; softmax is exact (max-subtracted). */
void orc_gqa_attention(const double *q, int64_t n_q_heads, int64_t n_kv_heads, int64_t hd,
                       const double *keys, const double *values, int64_t n_pos,
                       int64_t window, double scale, double *o, double *bound) {
    int64_t group = n_q_heads / n_kv_heads;
    int64_t lo = (window > 0 && n_pos > window) ? n_pos - window : 0;
    int64_t cnt = n_pos - lo;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)cnt);
        double *sa = (double *)malloc(sizeof(double) * (size_t)cnt);
#pragma omp for schedule(static)
        for (int64_t h = 0; h < n_q_heads; ++h) {
            int64_t g = h / group;
            const double *qh = q + h * hd;
            double m = -INFINITY;
            for (int64_t j = 0; j < cnt; ++j) {
                const double *kj = keys + ((lo + j) * n_kv_heads + g) * hd;
                double dot = 0.0, adot = 0.0;
                for (int64_t i = 0; i < hd; ++i) {
                    dot += qh[i] * kj[i];
                    adot += fabs(qh[i] * kj[i]);
                }
                s[j] = scale * dot;
                sa[j] = fabs(scale) * adot;
                if (s[j] > m)
                    m = s[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < cnt; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            for (int64_t j = 0; j < cnt; ++j)
                s[j] /= z; /* s now holds the softmax weights p_j */
            for (int64_t d = 0; d < hd; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < cnt; ++j)
                    acc += s[j] * values[((lo + j) * n_kv_heads + g) * hd + d];
                o[h * hd + d] = acc;
            }
            if (bound) {
                for (int64_t d = 0; d < hd; ++d) {
                    double a = 0.0, b = 0.0;
                    for (int64_t j = 0; j < cnt; ++j) {
                        double v = values[((lo + j) * n_kv_heads + g) * hd + d];
                        a += s[j] * fabs(v);
                        b += s[j] * fabs(v - o[h * hd + d]) * sa[j];
                    }
                    bound[h * hd + d] = a + b;
                }
            }
        }
        free(s);
        free(sa);
    }
}

/* Cache element i of a layer's cache: fp32, or binary16 (kv_f16). */
static double cache_load(const orc_layer *L, const void *c, int64_t i) {
    if (L->kv_f16) return orc_half_to_double(((const uint16_t *)c)[i]);
    return (double)((const float *)c)[i];
}
static void cache_store(const orc_layer *L, void *c, int64_t i, double v) {
    if (L->kv_f16)
        ((uint16_t *)c)[i] = orc_double_to_half(v);
    else
        ((float *)c)[i] = (float)v;
}

/* x += rmsnorm(y) * w, row by row (a post-norm joining the residual). */
static void post_norm_add(double *x, const double *y, const double *w, int64_t B, int64_t D,
                          double eps) {
    double *t = (double *)malloc(sizeof(double) * (size_t)(B * D));
    orc_rmsnorm(y, w, B, D, eps, t);
    for (int64_t i = 0; i < B * D; ++i)
        x[i] += t[i];
    free(t);
}

/* One decode step.  Block topology ([GELO] 06 Compute flow: pre-LN block,
 * QKV projection, per-head QK-norm before RoPE, GQA attention over the cache
 * plus the new row, O projection with residual, pre-FFN norm, gate/up,
 * SwiGLU, down projection with residual; tied LM head; greedy choice).
 * Gemma-4 full-attention layers take V from the K projection: the cached V
 * row is the unit-gain RMSNorm of the raw K row ([GEM] Verified model facts). */
void orc_decode_step(const orc_model *m, int64_t pos, const int32_t *tok, int32_t *next,
                     double *logits, double *margins) {
    int64_t B = m->batch, D = m->d_model, Hq = m->n_q_heads, F = m->ffn;
    double *x = (double *)malloc(sizeof(double) * (size_t)(B * D));
    double *xn = (double *)malloc(sizeof(double) * (size_t)(B * D));
    orc_q8_0_gather(m->embed, m->vocab, D, tok, B, x);
    if (m->embed_scale != 0.0)  /* Gemma: the gathered rows are scaled (by sqrt(d)) */
        for (int64_t i = 0; i < B * D; ++i)
            x[i] *= m->embed_scale;

    for (int64_t l = 0; l < m->n_layers; ++l) {
        const orc_layer *L = &m->layers[l];
        int64_t hd = L->head_dim, Hkv = L->n_kv_heads;
        int64_t nq = Hq * hd, nk = Hkv * hd, nv = L->v_from_k ? 0 : nk;
        /* p-RoPE ([GELO] generation page, glossary: only the first p * d_head
         * dims rotate, the rest pass through): the first rot dims rotate as a
         * NeoX rotation of a rot-dimensional vector */
        int64_t rot = L->rope_dims > 0 ? L->rope_dims : hd;
        int64_t nqkv = nq + nk + nv;
        double *qkv = (double *)malloc(sizeof(double) * (size_t)(B * nqkv));
        double *att = (double *)malloc(sizeof(double) * (size_t)(B * nq));

        orc_rmsnorm(x, L->attn_norm, B, D, m->eps, xn);
        orc_q4_0_matvec(L->wqkv, nqkv, D, xn, B, NULL, qkv, NULL);

        int64_t n_pos = pos + 1;
        int64_t lo = (L->window > 0 && n_pos > L->window) ? n_pos - L->window : 0;
        double *keys = (double *)malloc(sizeof(double) * (size_t)(n_pos * nk));
        double *vals = (double *)malloc(sizeof(double) * (size_t)(n_pos * nk));
        double *tmp = (double *)malloc(sizeof(double) * (size_t)hd);
        double *vrow = (double *)malloc(sizeof(double) * (size_t)hd);
        for (int64_t bi = 0; bi < B; ++bi) {
            double *q = qkv + bi * nqkv;
            double *kr = q + nq;
            double *vr = L->v_from_k ? NULL : kr + nk;
            for (int64_t h = 0; h < Hq; ++h) {
                orc_rmsnorm(q + h * hd, L->q_norm, 1, hd, m->eps, tmp);
                orc_rope_neox(tmp, rot, pos, L->rope_theta);
                memcpy(q + h * hd, tmp, sizeof(double) * (size_t)hd);
            }
            for (int64_t g = 0; g < Hkv; ++g) {
                if (L->v_from_k)
                    orc_rmsnorm(kr + g * hd, NULL, 1, hd, m->eps, vrow);
                else
                    memcpy(vrow, vr + g * hd, sizeof(double) * (size_t)hd);
                orc_rmsnorm(kr + g * hd, L->k_norm, 1, hd, m->eps, tmp);
                orc_rope_neox(tmp, rot, pos, L->rope_theta);
                /* the appended row is stored rounded to the cache's
                 * element type (fp32, or the nearest binary16) */
                int64_t slot = pos % L->cap;
                int64_t at = ((bi * Hkv + g) * L->cap + slot) * hd;
                for (int64_t i = 0; i < hd; ++i) {
                    cache_store(L, L->k_cache, at + i, tmp[i]);
                    cache_store(L, L->v_cache, at + i, vrow[i]);
                }
            }
            for (int64_t p = lo; p < n_pos; ++p) {
                int64_t slot = p % L->cap;
                for (int64_t g = 0; g < Hkv; ++g)
                    for (int64_t i = 0; i < hd; ++i) {
                        keys[(p * Hkv + g) * hd + i] =
                            cache_load(L, L->k_cache, ((bi * Hkv + g) * L->cap + slot) * hd + i);
                        vals[(p * Hkv + g) * hd + i] =
                            cache_load(L, L->v_cache, ((bi * Hkv + g) * L->cap + slot) * hd + i);
                    }
            }
            orc_gqa_attention(q, Hq, Hkv, hd, keys, vals, n_pos, L->window, L->attn_scale,
                              att + bi * nq, NULL);
        }
        free(keys);
        free(vals);
        free(tmp);
        free(vrow);

        /* sandwich norms ([GEM] 31B trace: post-attention RMSNorm, residual
         * add, FFN RMSNorm): with a post-norm gain the sublayer output is
         * RMS-normalised before it joins the residual */
        if (L->post_attn_norm) {
            orc_q4_0_matvec(L->wo, D, nq, att, B, NULL, xn, NULL);
            post_norm_add(x, xn, L->post_attn_norm, B, D, m->eps);
        } else {
            orc_q4_0_matvec(L->wo, D, nq, att, B, x, xn, NULL);
            memcpy(x, xn, sizeof(double) * (size_t)(B * D));
        }

        double *gu = (double *)malloc(sizeof(double) * (size_t)(B * 2 * F));
        double *hh = (double *)malloc(sizeof(double) * (size_t)(B * F));
        orc_rmsnorm(x, L->ffn_norm, B, D, m->eps, xn);
        orc_q4_0_matvec(L->wgu, 2 * F, D, xn, B, NULL, gu, NULL);
        for (int64_t bi = 0; bi < B; ++bi) {
            if (m->ffn_act == 1)
                orc_geglu(gu + bi * 2 * F, gu + bi * 2 * F + F, F, hh + bi * F);
            else
                orc_swiglu(gu + bi * 2 * F, gu + bi * 2 * F + F, F, hh + bi * F);
        }
        if (L->post_ffn_norm) {
            orc_q4_0_matvec(L->wd, D, F, hh, B, NULL, xn, NULL);
            post_norm_add(x, xn, L->post_ffn_norm, B, D, m->eps);
        } else {
            orc_q4_0_matvec(L->wd, D, F, hh, B, x, xn, NULL);
            memcpy(x, xn, sizeof(double) * (size_t)(B * D));
        }
        free(gu);
        free(hh);
        free(qkv);
        free(att);
    }

    orc_rmsnorm(x, m->final_norm, B, D, m->eps, xn);
    double *lg = logits ? logits : (double *)malloc(sizeof(double) * (size_t)(B * m->vocab));
    orc_q8_0_matvec(m->embed, m->vocab, D, xn, B, NULL, lg, NULL);
    if (m->logit_softcap > 0.0)
        orc_softcap(lg, B * m->vocab, m->logit_softcap);
    for (int64_t bi = 0; bi < B; ++bi) {
        double mg;
        next[bi] = (int32_t)orc_argmax(lg + bi * m->vocab, m->vocab, &mg);
        if (margins)
            margins[bi] = mg;
    }
    if (!logits)
        free(lg);
    free(x);
    free(xn);
}
