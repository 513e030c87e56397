// Decode scheduler: one autoregressive step of a pre-norm decoder, enqueued
// kernel by kernel or replayed as one captured HIP graph.
//
// Step topology ("GELO LLM" page, 06 "Compute flow & trust boundaries": per
// block RMSNorm, merged QKV projection, per-head QK-norm before RoPE, cached
// GQA attention, O projection with residual, RMSNorm, merged gate|up, SwiGLU,
// down projection with residual; 04: tied input/output embeddings; 05: greedy
// sampler).  The whole token is one command span and every buffer stays
// resident ("Research record" page, "Native Metal diagnostic: buffer
// ownership": persistent buffers and longer command spans).
//
// The position of the next token and n = position + 1 live in device memory
// and are advanced by the step's last kernel, so a graph captured once is
// valid for every later step.
//
// Sandwich post-norms (Gemma-4 block variant, "Research record" page, 31B
// trace: post-sublayer RMSNorm before the residual add) are applied by the
// next pre-normed projection where the vector kernels take them, so they cost
// no launch of their own; the residual stream then alternates between two
// buffers, since that projection's workgroups read the old stream while one
// of them writes the new one.
#include <vector>

#include "common.hpp"

struct q4_decode_model {
    q4_model_desc desc;
    std::vector<q4_layer_desc> layers;
    std::vector<q4_kv_layout> kv;
    int64_t *pos_dev = nullptr;  // [0] = position of the next token, [1] = n = position + 1
    float *x = nullptr, *qkv = nullptr, *att = nullptr, *gu = nullptr;
    float *tmp = nullptr;  // a sublayer output before its sandwich post-norm [B][d_model]
    float *x2 = nullptr;   // the residual stream's second buffer (fused post-norms) [B][d_model]
    void *arg = nullptr;  // the two-pass argmax's partial maxima
    float *logits = nullptr;
    void *attn_ws = nullptr;
    size_t attn_ws_bytes = 0;
    void *mv_ws = nullptr;  // matrix-core matvec workspace (batch >= 2), else NULL
    size_t mv_ws_bytes = 0;
    hipStream_t capture = nullptr;
    struct Graph {
        const int32_t *tok;
        int32_t *next;
        float *logits;
        hipGraphExec_t exec;
    };
    std::vector<Graph> graphs;
    int64_t pos_host = 0;
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kMaxGraphs = 4;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

__global__ void set_position_kernel(int64_t *pos, int64_t p) {
    pos[0] = p;
    pos[1] = p + 1;
}

__global__ void advance_position_kernel(int64_t *pos) {
    const int64_t p = pos[0] + 1;
    pos[0] = p;
    pos[1] = p + 1;
}

struct Layout {
    size_t pos, x, qkv, att, gu, logits, tmp, x2, arg, mv, mv_bytes, attn, total;
};

int64_t layer_qkv_rows(const q4_model_desc &d, const q4_layer_desc &l) {
    const int64_t nq = d.n_q_heads * l.head_dim, nk = l.n_kv_heads * l.head_dim;
    return nq + nk + (l.v_from_k ? 0 : nk);
}

q4_kv_layout layer_kv(const q4_model_desc &d, const q4_layer_desc &l) {
    q4_kv_layout kv;
    kv.batch = d.batch;
    kv.n_kv_heads = l.n_kv_heads;
    kv.head_dim = l.head_dim;
    kv.cap = l.cap;
    kv.stride_t = l.head_dim;
    kv.stride_h = l.cap * l.head_dim;
    kv.stride_b = l.n_kv_heads * l.cap * l.head_dim;
    kv.dtype = l.kv_dtype;
    return kv;
}

// With two or more sequences the projections run on the matrix cores
// (q4_0_matvec_batched) wherever the shape allows it.
bool batched_ok(const q4_model_desc &d, const void *W, int64_t K) {
    return d.batch >= 2 && K % 256 == 0 && q4::aligned(W, 16);
}

Layout plan(const q4_model_desc &d) {
    const int64_t B = d.batch;
    int64_t qkv = 0, att = 0;
    size_t attn = 0, mv = 0;
    auto need_mv = [&](const void *W, int64_t N, int64_t K) {
        if (batched_ok(d, W, K)) mv = std::max(mv, matvec_batched_workspace(N, K, B));
    };
    for (int64_t i = 0; i < d.n_layers; ++i) {
        const q4_layer_desc &l = d.layers[i];
        qkv = std::max(qkv, layer_qkv_rows(d, l));
        att = std::max(att, d.n_q_heads * l.head_dim);
        q4_kv_layout kv = layer_kv(d, l);
        attn = std::max(attn, gqa_decode_attn_workspace(&kv, d.n_q_heads, l.window));
        need_mv(l.wqkv, layer_qkv_rows(d, l), d.d_model);
        need_mv(l.wo, d.d_model, d.n_q_heads * l.head_dim);
        need_mv(l.wgu, 2 * d.ffn, d.d_model);
        need_mv(l.wd, d.d_model, d.ffn);
    }
    need_mv(d.embed, d.vocab, d.d_model);
    Layout L;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.pos = take(2 * sizeof(int64_t));
    L.x = take(sizeof(float) * B * d.d_model);
    L.qkv = take(sizeof(float) * B * qkv);
    L.att = take(sizeof(float) * B * att);
    L.gu = take(sizeof(float) * B * 2 * d.ffn);
    L.logits = take(sizeof(float) * B * d.vocab);
    L.tmp = take(sizeof(float) * B * d.d_model);
    L.x2 = take(sizeof(float) * B * d.d_model);
    L.arg = take(q4::argmax_scratch_bytes(B));
    L.mv = take(mv);
    L.mv_bytes = mv;
    L.attn = take(attn);
    L.total = o;
    return L;
}

q4_status validate(const q4_model_desc *d) {
    Q4_CHECK(d, Q4_ERR_INVALID_ARG, "decode model: desc must not be NULL");
    Q4_CHECK(d->n_layers >= 1 && d->layers, Q4_ERR_INVALID_ARG, "decode model: no layers");
    Q4_CHECK(d->embed && d->final_norm, Q4_ERR_INVALID_ARG, "decode model: embed and final_norm required");
    Q4_CHECK(d->d_model >= 32 && d->n_q_heads >= 1 && d->ffn >= 32 && d->vocab >= 1, Q4_ERR_INVALID_ARG,
             "decode model: sizes must be positive");
    Q4_CHECK(d->batch >= 1, Q4_ERR_INVALID_ARG, "decode model: batch must be >= 1");
    Q4_CHECK(d->batch <= 32, Q4_ERR_UNSUPPORTED, "decode model: batch %lld > 32", (long long)d->batch);
    // Beyond 8 sequences only the matrix-core projections apply.
    const bool wide = d->batch > 8;
    Q4_CHECK(!wide || (d->d_model % 256 == 0 && d->ffn % 256 == 0 && q4::aligned(d->embed, 16)),
             Q4_ERR_UNSUPPORTED,
             "decode model: batch %lld > 8 needs d_model and ffn multiples of 256 and a 16-byte aligned table",
             (long long)d->batch);
    Q4_CHECK(d->d_model % 32 == 0 && d->ffn % 32 == 0, Q4_ERR_SHAPE,
             "decode model: d_model and ffn must be multiples of 32");
    Q4_CHECK(d->eps >= 0.f, Q4_ERR_INVALID_ARG, "decode model: eps must be >= 0");
    Q4_CHECK(d->ffn_act == 0 || d->ffn_act == 1, Q4_ERR_INVALID_ARG,
             "decode model: ffn_act %d is neither 0 (SwiGLU) nor 1 (GeGLU)", (int)d->ffn_act);
    Q4_CHECK(d->embed_scale >= 0.f && d->embed_scale <= 1e30f && d->logit_softcap >= 0.f &&
                 d->logit_softcap <= 1e30f,
             Q4_ERR_INVALID_ARG, "decode model: embed_scale and logit_softcap must be finite and >= 0");
    for (int64_t i = 0; i < d->n_layers; ++i) {
        const q4_layer_desc &l = d->layers[i];
        Q4_CHECK(l.wqkv && l.wo && l.wgu && l.wd && l.attn_norm && l.ffn_norm && l.q_norm && l.k_norm &&
                     l.k_cache && l.v_cache,
                 Q4_ERR_INVALID_ARG, "decode model: layer %lld has a NULL pointer", (long long)i);
        Q4_CHECK(l.n_kv_heads >= 1 && d->n_q_heads % l.n_kv_heads == 0, Q4_ERR_SHAPE,
                 "decode model: layer %lld: n_q_heads not a multiple of n_kv_heads", (long long)i);
        Q4_CHECK(l.head_dim == 64 || l.head_dim == 128 || l.head_dim == 256 || l.head_dim == 512,
                 Q4_ERR_UNSUPPORTED, "decode model: layer %lld: head_dim %lld", (long long)i,
                 (long long)l.head_dim);
        Q4_CHECK(d->n_q_heads / l.n_kv_heads <= 16, Q4_ERR_UNSUPPORTED,
                 "decode model: layer %lld: more than 16 query heads per kv head", (long long)i);
        Q4_CHECK(l.cap >= 1 && l.window >= 0 && l.rope_theta > 0.0, Q4_ERR_INVALID_ARG,
                 "decode model: layer %lld: cap >= 1, window >= 0, rope_theta > 0", (long long)i);
        Q4_CHECK(l.kv_dtype == Q4_KV_F32 || l.kv_dtype == Q4_KV_F16, Q4_ERR_INVALID_ARG,
                 "decode model: layer %lld: kv_dtype %d unknown", (long long)i, (int)l.kv_dtype);
        Q4_CHECK(l.rope_dims == 0 || (l.rope_dims >= 2 && l.rope_dims <= l.head_dim && l.rope_dims % 2 == 0),
                 Q4_ERR_INVALID_ARG, "decode model: layer %lld: rope_dims %lld must be 0 or even in [2, head_dim]",
                 (long long)i, (long long)l.rope_dims);
        Q4_CHECK((!l.post_attn_norm || q4::aligned(l.post_attn_norm, 4)) &&
                     (!l.post_ffn_norm || q4::aligned(l.post_ffn_norm, 4)),
                 Q4_ERR_ALIGNMENT, "decode model: layer %lld: post-norm gains must be 4-byte aligned",
                 (long long)i);
        Q4_CHECK(q4::aligned(l.k_cache, 16) && q4::aligned(l.v_cache, 16) && q4::aligned(l.wqkv, 2) &&
                     q4::aligned(l.wo, 2) && q4::aligned(l.wgu, 2) && q4::aligned(l.wd, 2) &&
                     q4::aligned(l.attn_norm, 4) && q4::aligned(l.ffn_norm, 4) &&
                     q4::aligned(l.q_norm, 4) && q4::aligned(l.k_norm, 4),
                 Q4_ERR_ALIGNMENT, "decode model: layer %lld: caches need 16-byte, weights 2-byte, norms 4-byte alignment",
                 (long long)i);
        Q4_CHECK((d->n_q_heads * l.head_dim) % 32 == 0, Q4_ERR_SHAPE,
                 "decode model: layer %lld: n_q_heads * head_dim must be a multiple of 32", (long long)i);
        Q4_CHECK(!wide || ((d->n_q_heads * l.head_dim) % 256 == 0 && q4::aligned(l.wqkv, 16) &&
                           q4::aligned(l.wo, 16) && q4::aligned(l.wgu, 16) && q4::aligned(l.wd, 16)),
                 Q4_ERR_UNSUPPORTED,
                 "decode model: layer %lld: batch > 8 needs n_q_heads * head_dim a multiple of 256 "
                 "and 16-byte aligned weights", (long long)i);
    }
    return Q4_OK;
}

bool fits(const q4_decode_model *m, int64_t pos) {
    for (const q4_layer_desc &l : m->layers)
        if (!(l.cap >= pos + 1 || (l.window > 0 && l.cap >= l.window))) return false;
    return true;
}

#define Q4_TRY(expr)                          \
    do {                                      \
        q4_status s_ = (expr);                \
        if (s_ != Q4_OK) return s_;           \
    } while (0)

// One projection of the step: matrix cores for two or more sequences,
// otherwise the vector-unit kernels.
q4_status project(q4_decode_model *m, int fmt, const void *W, int64_t N, int64_t K, const float *x,
                  const float *x2, int64_t ldx, q4_input_op op, q4_output_op out, const float *nw,
                  float *y, const float *res, void *s) {
    const q4_model_desc &d = m->desc;
    if (m->mv_ws && batched_ok(d, W, K))
        return (fmt == 0 ? q4_0_matvec_batched : q8_0_matvec_batched)(
            W, N, K, x, x2, ldx, d.batch, op, out, nw, d.eps, y, res, m->mv_ws, m->mv_ws_bytes, s);
    return (fmt == 0 ? q4_0_matvec_fused : q8_0_matvec_fused)(W, N, K, x, x2, ldx, d.batch, op, out,
                                                              nw, d.eps, y, res, s);
}

// A waiting post-norm can be fused into a pre-normed Q4_0 projection on the
// vector kernels (q4_0_matvec_post_norm: up to 8 rows, K % 256 == 0,
// K <= 8192, 16-byte aligned gains).
bool post_fusable(const q4_decode_model *m, const void *W, const float *post_w, const float *pre_w) {
    const q4_model_desc &d = m->desc;
    return !(m->mv_ws && batched_ok(d, W, d.d_model)) && d.batch <= 8 && d.d_model % 256 == 0 &&
           d.d_model <= 8192 && q4::aligned(post_w, 16) && (!pre_w || q4::aligned(pre_w, 16));
}

// The gate|up projection can hand SiLU(gate) * up straight to the down
// projection when its kernel supports a SwiGLU output for this shape.
bool glu_output(const q4_model_desc &d, const void *wgu) {
    if (batched_ok(d, wgu, d.d_model)) return true;
    return d.d_model % 256 == 0 && d.d_model <= 8192;
}

// Enqueues one whole step on s.
q4_status enqueue_step(q4_decode_model *m, const int32_t *tok, int32_t *next, float *logits,
                       hipStream_t s) {
    const q4_model_desc &d = m->desc;
    const int64_t B = d.batch, D = d.d_model, F = d.ffn;
    void *sv = s;
    if (d.embed_scale != 0.f && d.embed_scale != 1.f)
        Q4_TRY(q8_0_gather_scaled(d.embed, d.vocab, D, tok, B, d.embed_scale, m->x, sv));
    else
        Q4_TRY(q8_0_gather(d.embed, d.vocab, D, tok, B, m->x, sv));
    const q4_input_op gated_in = d.ffn_act ? Q4_IN_GEGLU : Q4_IN_SWIGLU;
    const q4_output_op gated_out = d.ffn_act ? Q4_OUT_GEGLU : Q4_OUT_SWIGLU;
    // The residual stream lives in hc.  A sandwich post-norm whose sublayer
    // output waits in tmp (gain pend) joins the stream inside the next
    // pre-normed projection where the vector kernels can take it, writing the
    // stream's other buffer; otherwise rmsnorm_add applies it in place first.
    float *hc = m->x, *ha = m->x2;
    const float *pend = nullptr;
    auto normed_proj = [&](const void *W, int64_t N, const float *gain, q4_output_op out,
                           float *y) -> q4_status {
        if (pend && post_fusable(m, W, pend, gain)) {
            Q4_TRY(q4_0_matvec_post_norm(W, N, D, hc, m->tmp, D, B, pend, gain, d.eps, ha, out, y, sv));
            std::swap(hc, ha);
            pend = nullptr;
            return Q4_OK;
        }
        if (pend) Q4_TRY(rmsnorm_add(m->tmp, pend, B, D, d.eps, hc, sv));
        pend = nullptr;
        return project(m, 0, W, N, D, hc, nullptr, D, Q4_IN_RMSNORM, out, gain, y, nullptr, sv);
    };
    for (size_t i = 0; i < m->layers.size(); ++i) {
        const q4_layer_desc &l = m->layers[i];
        const int64_t hd = l.head_dim, nq = d.n_q_heads * hd, nk = l.n_kv_heads * hd;
        const int64_t nqkv = layer_qkv_rows(d, l);
        // attention RMSNorm fused into the QKV projection's input
        Q4_TRY(normed_proj(l.wqkv, nqkv, l.attn_norm, Q4_OUT_PLAIN, m->qkv));
        if (l.rope_dims == 0 || l.rope_dims == hd) {
            // per-head QK-norm, RoPE and the KV append fused into the attention
            Q4_TRY(gqa_decode_attn_rope(m->qkv, nqkv, d.n_q_heads, l.q_norm, l.k_norm, &m->kv[i],
                                        m->pos_dev, l.rope_theta, d.eps, l.v_from_k, l.k_cache,
                                        l.v_cache, l.window, l.attn_scale, m->att, nq, m->attn_ws,
                                        m->attn_ws_bytes, sv));
        } else {
            // p-RoPE: the standalone preparation (q in place, the append),
            // then attention over n = pos + 1 positions
            Q4_TRY(qk_norm_rope_partial(m->qkv, nqkv, m->qkv + nq,
                                        l.v_from_k ? nullptr : m->qkv + nq + nk, nqkv, l.q_norm,
                                        l.k_norm, d.n_q_heads, &m->kv[i], m->pos_dev, l.rope_theta,
                                        d.eps, l.v_from_k, l.rope_dims, l.k_cache, l.v_cache, sv));
            Q4_TRY(gqa_decode_attn(m->qkv, nqkv, d.n_q_heads, l.k_cache, l.v_cache, &m->kv[i],
                                   m->pos_dev + 1, l.window, l.attn_scale, m->att, nq, m->attn_ws,
                                   m->attn_ws_bytes, sv));
        }
        // O projection; with a sandwich post-norm the output is normalised
        // before it joins the residual
        if (l.post_attn_norm) {
            Q4_TRY(project(m, 0, l.wo, D, nq, m->att, nullptr, nq, Q4_IN_PLAIN, Q4_OUT_PLAIN, nullptr,
                           m->tmp, nullptr, sv));
            pend = l.post_attn_norm;
        } else {
            Q4_TRY(project(m, 0, l.wo, D, nq, m->att, nullptr, nq, Q4_IN_PLAIN, Q4_OUT_PLAIN, nullptr,
                           hc, hc, sv));
        }
        // FFN RMSNorm fused into gate|up; SwiGLU fused into gate|up's output
        // (else into the down projection's input)
        const bool gout = glu_output(d, l.wgu);
        Q4_TRY(normed_proj(l.wgu, 2 * F, l.ffn_norm, gout ? gated_out : Q4_OUT_PLAIN, m->gu));
        float *dy = l.post_ffn_norm ? m->tmp : hc;          // down projection output
        const float *dres = l.post_ffn_norm ? nullptr : hc;  // and its residual
        if (gout)
            Q4_TRY(project(m, 0, l.wd, D, F, m->gu, nullptr, F, Q4_IN_PLAIN, Q4_OUT_PLAIN, nullptr,
                           dy, dres, sv));
        else
            Q4_TRY(project(m, 0, l.wd, D, F, m->gu, m->gu + F, 2 * F, gated_in, Q4_OUT_PLAIN,
                           nullptr, dy, dres, sv));
        if (l.post_ffn_norm) pend = l.post_ffn_norm;
    }
    if (pend) Q4_TRY(rmsnorm_add(m->tmp, pend, B, D, d.eps, hc, sv));
    float *lg = logits ? logits : m->logits;
    Q4_TRY(project(m, 1, d.embed, d.vocab, D, hc, nullptr, D, Q4_IN_RMSNORM, Q4_OUT_PLAIN,
                   d.final_norm, lg, nullptr, sv));
    if (d.logit_softcap > 0.f) Q4_TRY(softcap(lg, B * d.vocab, d.logit_softcap, sv));
    Q4_TRY(q4::argmax_rows_scratch(lg, B, d.vocab, next, m->arg, s));
    hipLaunchKernelGGL(advance_position_kernel, dim3(1), dim3(1), 0, s, m->pos_dev);
    return q4::launch_status("decode_step (advance)");
}

q4_status check_step_args(q4_decode_model *m, const int32_t *tok, int32_t *next, float *logits) {
    Q4_CHECK(m, Q4_ERR_INVALID_ARG, "decode_step: model must not be NULL");
    Q4_CHECK(tok && next, Q4_ERR_INVALID_ARG, "decode_step: tokens and next_tokens must not be NULL");
    Q4_CHECK(q4::aligned(tok, 4) && q4::aligned(next, 4) && (!logits || q4::aligned(logits, 4)),
             Q4_ERR_ALIGNMENT, "decode_step: tokens, next and logits must be 4-byte aligned");
    Q4_CHECK(fits(m, m->pos_host), Q4_ERR_CAPACITY,
             "decode_step: position %lld does not fit a layer's KV cache", (long long)m->pos_host);
    return Q4_OK;
}

}  // namespace

extern "C" q4_status decode_model_workspace(const q4_model_desc *desc, size_t *bytes) {
    q4::clear_error();
    Q4_CHECK(bytes, Q4_ERR_INVALID_ARG, "decode_model_workspace: bytes must not be NULL");
    q4_status st = validate(desc);
    if (st != Q4_OK) return st;
    *bytes = plan(*desc).total;
    return Q4_OK;
}

extern "C" q4_status decode_model_create(const q4_model_desc *desc, void *ws, size_t ws_bytes,
                                         q4_decode_model **out) {
    q4::clear_error();
    Q4_CHECK(out, Q4_ERR_INVALID_ARG, "decode_model_create: out must not be NULL");
    *out = nullptr;
    q4_status st = validate(desc);
    if (st != Q4_OK) return st;
    const Layout L = plan(*desc);
    Q4_CHECK(ws && ws_bytes >= L.total, Q4_ERR_WORKSPACE,
             "decode_model_create: workspace of %zu bytes needed, got %zu", L.total, ws_bytes);
    Q4_CHECK(q4::aligned(ws, kAlign), Q4_ERR_ALIGNMENT,
             "decode_model_create: workspace must be 256-byte aligned");
    q4_decode_model *m = new q4_decode_model();
    m->desc = *desc;
    m->layers.assign(desc->layers, desc->layers + desc->n_layers);
    m->desc.layers = m->layers.data();
    for (const q4_layer_desc &l : m->layers) m->kv.push_back(layer_kv(*desc, l));
    char *base = static_cast<char *>(ws);
    m->pos_dev = reinterpret_cast<int64_t *>(base + L.pos);
    m->x = reinterpret_cast<float *>(base + L.x);
    m->qkv = reinterpret_cast<float *>(base + L.qkv);
    m->att = reinterpret_cast<float *>(base + L.att);
    m->gu = reinterpret_cast<float *>(base + L.gu);
    m->logits = reinterpret_cast<float *>(base + L.logits);
    m->tmp = reinterpret_cast<float *>(base + L.tmp);
    m->x2 = reinterpret_cast<float *>(base + L.x2);
    m->arg = base + L.arg;
    m->attn_ws = base + L.attn;
    m->attn_ws_bytes = L.total - L.attn;
    m->mv_ws = L.mv_bytes ? base + L.mv : nullptr;
    m->mv_ws_bytes = L.mv_bytes;
    hipError_t e = hipStreamCreateWithFlags(&m->capture, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete m;
        return q4::fail(Q4_ERR_HIP, "decode_model_create: hipStreamCreate: %s", hipGetErrorString(e));
    }
    hipLaunchKernelGGL(set_position_kernel, dim3(1), dim3(1), 0, m->capture, m->pos_dev, int64_t(0));
    e = hipGetLastError();
    // the matrix-core matvec's split tickets start at zero (each call leaves them so)
    if (e == hipSuccess && m->mv_ws) e = hipMemsetAsync(m->mv_ws, 0, m->mv_ws_bytes, m->capture);
    if (e == hipSuccess) e = hipStreamSynchronize(m->capture);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(m->capture);
        delete m;
        return q4::fail(Q4_ERR_HIP, "decode_model_create: %s", hipGetErrorString(e));
    }
    *out = m;
    return Q4_OK;
}

extern "C" q4_status decode_model_set_position(q4_decode_model *m, int64_t pos, void *stream) {
    q4::clear_error();
    Q4_CHECK(m, Q4_ERR_INVALID_ARG, "decode_model_set_position: model must not be NULL");
    Q4_CHECK(pos >= 0, Q4_ERR_INVALID_ARG, "decode_model_set_position: pos must be >= 0");
    Q4_CHECK(fits(m, pos), Q4_ERR_CAPACITY,
             "decode_model_set_position: position %lld does not fit a layer's KV cache", (long long)pos);
    hipLaunchKernelGGL(set_position_kernel, dim3(1), dim3(1), 0, q4::as_stream(stream), m->pos_dev, pos);
    q4_status st = q4::launch_status("decode_model_set_position");
    if (st == Q4_OK) m->pos_host = pos;
    return st;
}

extern "C" int64_t decode_model_position(const q4_decode_model *m) { return m ? m->pos_host : -1; }

extern "C" q4_status decode_step_eager(q4_decode_model *m, const int32_t *tokens_dev,
                                       int32_t *next_tokens_dev, float *logits_dev, void *stream) {
    q4::clear_error();
    q4_status st = check_step_args(m, tokens_dev, next_tokens_dev, logits_dev);
    if (st != Q4_OK) return st;
    st = enqueue_step(m, tokens_dev, next_tokens_dev, logits_dev, q4::as_stream(stream));
    if (st == Q4_OK) m->pos_host += 1;
    return st;
}

extern "C" q4_status decode_step(q4_decode_model *m, const int32_t *tokens_dev,
                                 int32_t *next_tokens_dev, float *logits_dev, void *stream) {
    q4::clear_error();
    q4_status st = check_step_args(m, tokens_dev, next_tokens_dev, logits_dev);
    if (st != Q4_OK) return st;
    hipGraphExec_t exec = nullptr;
    for (const auto &g : m->graphs)
        if (g.tok == tokens_dev && g.next == next_tokens_dev && g.logits == logits_dev) exec = g.exec;
    if (!exec) {
        Q4_HIP_CHECK(hipStreamBeginCapture(m->capture, hipStreamCaptureModeThreadLocal));
        st = enqueue_step(m, tokens_dev, next_tokens_dev, logits_dev, m->capture);
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamEndCapture(m->capture, &graph);
        if (st != Q4_OK) {
            if (graph) (void)hipGraphDestroy(graph);
            return st;
        }
        if (e != hipSuccess) return q4::fail(Q4_ERR_HIP, "decode_step: capture: %s", hipGetErrorString(e));
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess) return q4::fail(Q4_ERR_HIP, "decode_step: instantiate: %s", hipGetErrorString(e));
        if (m->graphs.size() >= kMaxGraphs) {
            (void)hipGraphExecDestroy(m->graphs.front().exec);
            m->graphs.erase(m->graphs.begin());
        }
        m->graphs.push_back({tokens_dev, next_tokens_dev, logits_dev, exec});
    }
    Q4_HIP_CHECK(hipGraphLaunch(exec, q4::as_stream(stream)));
    m->pos_host += 1;
    return Q4_OK;
}

extern "C" q4_status decode_model_destroy(q4_decode_model *m) {
    q4::clear_error();
    if (!m) return Q4_OK;
    for (auto &g : m->graphs) (void)hipGraphExecDestroy(g.exec);
    if (m->capture) (void)hipStreamDestroy(m->capture);
    delete m;
    return Q4_OK;
}
