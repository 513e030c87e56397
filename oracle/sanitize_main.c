/*
 * sanitize_main.c -- memory- and UB-checking driver for oracle.c.
 * TEST INFRASTRUCTURE ONLY.  Built with gcc -fsanitize=address,undefined by
 * the CPU test suite; it calls every oracle function on small seeded inputs
 * (ragged block tails, batches, NULL optional arguments, windows, binary16
 * caches, ring-buffer wrap in a decode loop) so that an out-of-bounds access
 * or undefined operation aborts the run.  Values are not checked here: the
 * pins in the Python tests do that.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) { /* xorshift64* */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static double uniform(double lo, double hi) { return lo + (hi - lo) * (next_u32() / 4294967296.0); }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* Q4_0 / Q8_0 rows with binary16 scales in [lo, hi] and random codes. */
static uint8_t *quant_rows(int64_t rows, int64_t k, int q8, double lo, double hi) {
    const int64_t bpb = q8 ? 34 : 18, nb = k / 32;
    uint8_t *w = xmalloc((size_t)(rows * nb * bpb));
    for (int64_t i = 0; i < rows * nb; ++i) {
        uint8_t *b = w + i * bpb;
        const uint16_t d = orc_double_to_half(uniform(lo, hi));
        b[0] = (uint8_t)(d & 0xFF);
        b[1] = (uint8_t)(d >> 8);
        for (int j = 2; j < bpb; ++j) b[j] = (uint8_t)next_u32();
    }
    return w;
}

static double *vec(int64_t n, double lo, double hi) {
    double *v = xmalloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) v[i] = uniform(lo, hi);
    return v;
}

static void check_basic_ops(void) {
    /* binary16 both ways, including specials */
    const uint16_t specials[] = {0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x7C00, 0xFC00, 0x7E00};
    for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i)
        (void)orc_double_to_half(orc_half_to_double(specials[i]));
    (void)orc_double_to_half(1e9);
    (void)orc_double_to_half(-1e-12);
    (void)orc_double_to_half(NAN);

    /* matvecs: ragged row counts, K of one and several blocks, batch 3, with
     * and without residual / terms */
    const int64_t shapes[][2] = {{1, 32}, {5, 64}, {7, 96}, {13, 256}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int64_t n = shapes[s][0], k = shapes[s][1], B = 3;
        for (int q8 = 0; q8 < 2; ++q8) {
            uint8_t *w = quant_rows(n, k, q8, 0.005, 0.02);
            double *x = vec(B * k, -2, 2), *res = vec(B * n, -1, 1);
            double *y = xmalloc((size_t)(B * n) * sizeof(double));
            double *t = xmalloc((size_t)(B * n) * sizeof(double));
            double *dq = xmalloc((size_t)(n * k) * sizeof(double));
            if (q8) {
                orc_q8_0_dequant(w, n, k, dq);
                orc_q8_0_matvec(w, n, k, x, B, res, y, t);
                orc_q8_0_matvec(w, n, k, x, 1, NULL, y, NULL);
                const int32_t tok[3] = {0, (int32_t)(n - 1), (int32_t)(n / 2)};
                double *g = xmalloc((size_t)(3 * k) * sizeof(double));
                orc_q8_0_gather(w, n, k, tok, 3, g);
                free(g);
            } else {
                orc_q4_0_dequant(w, n, k, dq);
                orc_q4_0_matvec(w, n, k, x, B, res, y, t);
                orc_q4_0_matvec(w, n, k, x, 1, NULL, y, NULL);
            }
            free(w), free(x), free(res), free(y), free(t), free(dq);
        }
    }

    /* elementwise ops */
    double *a = vec(37, -4, 4), *b = vec(37, -4, 4), *h = vec(37, 0, 1), *g = vec(37, 0.8, 1.2);
    orc_rmsnorm(a, g, 1, 37, 1e-6, h);
    orc_rmsnorm(a, NULL, 1, 37, 1e-6, h);
    orc_swiglu(a, b, 37, h);
    orc_geglu(a, b, 37, h);
    orc_softcap(h, 37, 30.0);
    double margin;
    (void)orc_argmax(a, 37, &margin);
    (void)orc_argmax(a, 1, &margin);
    double *r = vec(16, -1, 1);
    orc_rope_neox(r, 16, 4097, 1e6);
    orc_rope_neox(r, 8, 3, 1e4); /* partial: first 8 of 16 */
    free(a), free(b), free(h), free(g), free(r);

    /* attention: GQA groups, window smaller and larger than the positions */
    const int64_t hq = 4, hkv = 2, hd = 16, npos = 11;
    double *q = vec(hq * hd, -1, 1), *keys = vec(npos * hkv * hd, -1, 1);
    double *vals = vec(npos * hkv * hd, -1, 1);
    double *o = xmalloc((size_t)(hq * hd) * sizeof(double));
    double *bound = xmalloc((size_t)(hq * hd) * sizeof(double));
    const int64_t windows[] = {0, 1, 4, 64};
    for (size_t i = 0; i < 4; ++i) orc_gqa_attention(q, hq, hkv, hd, keys, vals, npos, windows[i], 0.25, o, bound);
    orc_gqa_attention(q, hq, hkv, hd, keys, vals, 1, 0, 0.25, o, NULL);
    free(q), free(keys), free(vals), free(o), free(bound);
}

/* A tiny decoder: a full fp32 layer, a sliding-window layer with binary16
 * caches shorter than the steps run (ring wrap), and a full layer with V from
 * K, partial RoPE and sandwich norms; GeGLU, scaled embedding, softcap. */
static void check_decode(void) {
    const int64_t d = 64, hq = 4, ffn = 96, vocab = 50, batch = 2, steps = 10;
    orc_layer L[3];
    memset(L, 0, sizeof(L));
    const int64_t hkv[3] = {2, 2, 1}, hdim[3] = {16, 16, 32}, cap[3] = {16, 4, 16}, win[3] = {0, 4, 0};
    const int32_t vfk[3] = {0, 0, 1}, f16[3] = {0, 1, 0};
    const int64_t rdims[3] = {0, 0, 16};
    void *owned[64];
    int no = 0;
    for (int l = 0; l < 3; ++l) {
        const int64_t hd = hdim[l], kvr = hkv[l] * hd;
        const int64_t qkv_rows = hq * hd + kvr + (vfk[l] ? 0 : kvr);
        L[l].wqkv = owned[no++] = quant_rows(qkv_rows, d, 0, 0.005, 0.02);
        L[l].wo = owned[no++] = quant_rows(d, hq * hd, 0, 0.005, 0.02);
        L[l].wgu = owned[no++] = quant_rows(2 * ffn, d, 0, 0.005, 0.02);
        L[l].wd = owned[no++] = quant_rows(d, ffn, 0, 0.005, 0.02);
        L[l].attn_norm = owned[no++] = vec(d, 0.8, 1.2);
        L[l].ffn_norm = owned[no++] = vec(d, 0.8, 1.2);
        L[l].q_norm = owned[no++] = vec(hd, 0.8, 1.2);
        L[l].k_norm = owned[no++] = vec(hd, 0.8, 1.2);
        const size_t cells = (size_t)(batch * hkv[l] * cap[l] * hd);
        const size_t esz = f16[l] ? 2 : 4;
        L[l].k_cache = owned[no++] = xmalloc(cells * esz);
        L[l].v_cache = owned[no++] = xmalloc(cells * esz);
        memset(L[l].k_cache, 0, cells * esz);
        memset(L[l].v_cache, 0, cells * esz);
        L[l].n_kv_heads = hkv[l];
        L[l].head_dim = hd;
        L[l].cap = cap[l];
        L[l].window = win[l];
        L[l].rope_theta = 1e4;
        L[l].attn_scale = 1.0 / sqrt((double)hd);
        L[l].v_from_k = vfk[l];
        L[l].kv_f16 = f16[l];
        L[l].rope_dims = rdims[l];
        if (l == 2) {
            L[l].post_attn_norm = owned[no++] = vec(d, 0.8, 1.2);
            L[l].post_ffn_norm = owned[no++] = vec(d, 0.8, 1.2);
        }
    }
    orc_model m;
    memset(&m, 0, sizeof(m));
    m.n_layers = 3;
    m.d_model = d;
    m.n_q_heads = hq;
    m.ffn = ffn;
    m.vocab = vocab;
    m.batch = batch;
    m.eps = 1e-6;
    m.embed = owned[no++] = quant_rows(vocab, d, 1, 0.002, 0.01);
    m.final_norm = owned[no++] = vec(d, 0.8, 1.2);
    m.layers = L;
    m.ffn_act = 1;
    m.embed_scale = 8.0;
    m.logit_softcap = 30.0;
    int32_t tok[2] = {3, 41}, nxt[2];
    double *logits = xmalloc((size_t)(batch * vocab) * sizeof(double));
    double margins[2];
    for (int64_t p = 0; p < steps; ++p) {
        orc_decode_step(&m, p, tok, nxt, (p & 1) ? NULL : logits, (p & 2) ? NULL : margins);
        tok[0] = nxt[0];
        tok[1] = nxt[1];
    }
    m.ffn_act = 0; /* the SwiGLU block too */
    m.embed_scale = 0.0;
    m.logit_softcap = 0.0;
    orc_decode_step(&m, steps, tok, nxt, logits, margins);
    free(logits);
    for (int i = 0; i < no; ++i) free(owned[i]);
}

int main(void) {
    check_basic_ops();
    check_decode();
    printf("oracle sanitize run: ok (%d threads)\n", orc_num_threads());
    return 0;
}
