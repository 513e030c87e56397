// Host-side checking driver of the C ABI (test infrastructure).  Built by the
// CPU test suite from the library sources with the host pass instrumented by
// AddressSanitizer and UndefinedBehaviorSanitizer (--cuda-host-only: no
// device code), and run on a machine without a GPU.  Every entry point is
// called with arguments its host validation must reject, and with valid,
// aligned arguments that pass validation and reach the HIP runtime, which
// has no device: those calls must return Q4_ERR_HIP.  No buffer here is
// ever dereferenced by a kernel.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "q4dec.h"

static int g_fail = 0;

static void expect(const char *what, q4_status got, q4_status want) {
    const char *msg = q4dec_last_error();
    if (got != want || (got != Q4_OK && (!msg || !msg[0]))) {
        std::fprintf(stderr, "FAIL %s: status %d (want %d): %s\n", what, got, want, msg ? msg : "");
        ++g_fail;
    }
}

static void expect_rejected(const char *what, q4_status got) {
    if (got == Q4_OK || got == Q4_ERR_HIP) {
        std::fprintf(stderr, "FAIL %s: not rejected on the host (status %d)\n", what, got);
        ++g_fail;
    }
}

int main() {
    // host buffers standing in for device ones (never touched by a kernel)
    std::vector<uint8_t> W(256 * 8 * 34 + 4096, 0);
    std::vector<float> x(32 * 8192 + 64, 0.f), y(32 * 8192 + 64, 0.f), g(8192, 1.f);
    std::vector<int32_t> tok(64, 0);
    std::vector<int64_t> pos(4, 0);
    void *w = W.data();
    float *xp = x.data(), *yp = y.data(), *gp = g.data();
    const int64_t N = 64, K = 256;

    // ---- matvec family
    expect_rejected("q4_0_matvec null W", q4_0_matvec(nullptr, N, K, xp, 1, yp, nullptr, nullptr));
    expect_rejected("q4_0_matvec K%32", q4_0_matvec(w, N, 48, xp, 1, yp, nullptr, nullptr));
    expect_rejected("q4_0_matvec B>8", q4_0_matvec(w, N, K, xp, 9, yp, nullptr, nullptr));
    expect_rejected("q4_0_matvec N=0", q4_0_matvec(w, 0, K, xp, 1, yp, nullptr, nullptr));
    expect_rejected("q8_0_matvec misaligned x", q8_0_matvec(w, N, K, xp + 0, 1, (float *)((char *)yp + 2), nullptr, nullptr));
    expect("q4_0_matvec valid", q4_0_matvec(w, N, K, xp, 2, yp, nullptr, nullptr), Q4_ERR_HIP);
    expect("q8_0_matvec valid", q8_0_matvec(w, N, K, xp, 1, yp, yp, nullptr), Q4_ERR_HIP);
    expect_rejected("fused ld<K", q4_0_matvec_fused(w, N, K, xp, nullptr, K - 32, 1, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                                                    nullptr, 0.f, yp, nullptr, nullptr));
    expect_rejected("fused swiglu without x2", q4_0_matvec_fused(w, N, K, xp, nullptr, K, 1, Q4_IN_SWIGLU,
                                                                 Q4_OUT_PLAIN, nullptr, 0.f, yp, nullptr, nullptr));
    expect("fused rmsnorm valid", q4_0_matvec_fused(w, N, K, xp, nullptr, K, 1, Q4_IN_RMSNORM, Q4_OUT_PLAIN, gp,
                                                    1e-6f, yp, nullptr, nullptr),
           Q4_ERR_HIP);
    expect("q8 fused valid", q8_0_matvec_fused(w, N, K, xp, nullptr, K, 1, Q4_IN_PLAIN, Q4_OUT_PLAIN, nullptr, 0.f,
                                               yp, nullptr, nullptr),
           Q4_ERR_HIP);
    expect_rejected("post_norm null h", q4_0_matvec_post_norm(w, N, K, nullptr, xp, K, 1, gp, gp, 1e-6f, yp,
                                                              Q4_OUT_PLAIN, yp, nullptr));
    size_t wsb = matvec_batched_workspace(N, K, 8);
    std::vector<uint8_t> wsv(wsb + 512);
    void *ws = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(wsv.data()) + 255) / 256 * 256);
    expect_rejected("batched B=33", q4_0_matvec_batched(w, N, K, xp, nullptr, K, 33, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                                                        nullptr, 0.f, yp, nullptr, ws, wsb, nullptr));
    expect_rejected("batched small ws", q4_0_matvec_batched(w, N, K, xp, nullptr, K, 8, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                                                            nullptr, 0.f, yp, nullptr, ws, 0, nullptr));
    expect("batched valid", q4_0_matvec_batched(w, N, K, xp, nullptr, K, 8, Q4_IN_PLAIN, Q4_OUT_PLAIN, nullptr, 0.f,
                                                 yp, nullptr, ws, wsb, nullptr),
           Q4_ERR_HIP);
    expect_rejected("q8 batched null y", q8_0_matvec_batched(w, N, K, xp, nullptr, K, 8, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                                                             nullptr, 0.f, nullptr, nullptr, ws, wsb, nullptr));
    expect_rejected("noalloc K%256", q4_0_matvec_batched_noalloc(w, N, 64, xp, nullptr, 64, 2, Q4_IN_PLAIN,
                                                                 Q4_OUT_PLAIN, nullptr, 0.f, yp, nullptr, nullptr));
    expect("noalloc valid", q4_0_matvec_batched_noalloc(w, N, K, xp, nullptr, K, 2, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                                                        nullptr, 0.f, yp, nullptr, nullptr),
           Q4_ERR_HIP);

    // ---- gather and elementwise
    expect_rejected("gather K%32", q8_0_gather(w, 10, 33, tok.data(), 1, xp, nullptr));
    expect("gather valid", q8_0_gather(w, 10, K, tok.data(), 2, xp, nullptr), Q4_ERR_HIP);
    expect("gather scaled valid", q8_0_gather_scaled(w, 10, K, tok.data(), 2, 2.f, xp, nullptr), Q4_ERR_HIP);
    expect_rejected("rmsnorm dim 0", rmsnorm(xp, gp, 1, 0, 1e-6f, yp, nullptr));
    expect("rmsnorm valid", rmsnorm(xp, gp, 2, K, 1e-6f, yp, nullptr), Q4_ERR_HIP);
    expect("rmsnorm_add valid", rmsnorm_add(yp, gp, 2, K, 1e-6f, xp, nullptr), Q4_ERR_HIP);
    expect_rejected("swiglu ld<n", swiglu(xp, yp, 2, K, K - 1, yp, nullptr));
    expect("swiglu valid", swiglu(xp, xp + K, 2, K, 2 * K, yp, nullptr), Q4_ERR_HIP);
    expect("geglu valid", geglu(xp, xp + K, 2, K, 2 * K, yp, nullptr), Q4_ERR_HIP);
    expect_rejected("softcap null", softcap(nullptr, 4, 30.f, nullptr));
    expect("softcap valid", softcap(yp, 64, 30.f, nullptr), Q4_ERR_HIP);

    // ---- attention side
    q4_kv_layout kv{};
    kv.batch = 2;
    kv.n_kv_heads = 2;
    kv.head_dim = 64;
    kv.cap = 32;
    kv.stride_t = 64;
    kv.stride_h = 32 * 64;
    kv.stride_b = 2 * 32 * 64;
    kv.dtype = Q4_KV_F32;
    std::vector<float> kc(2 * 2 * 32 * 64), vc(kc.size());
    q4_kv_layout bad = kv;
    bad.head_dim = 63;
    expect_rejected("qk_norm_rope odd hd", qk_norm_rope(xp, 4 * 64, xp, xp, 2 * 64, gp, gp, 4, &bad, pos.data(),
                                                        1e4, 1e-6f, 0, kc.data(), vc.data(), nullptr));
    expect("qk_norm_rope valid", qk_norm_rope(xp, 4 * 64, xp + 512, xp + 1024, 2 * 64, gp, gp, 4, &kv, pos.data(),
                                              1e4, 1e-6f, 0, kc.data(), vc.data(), nullptr),
           Q4_ERR_HIP);
    expect("qk_norm_rope_partial valid",
           qk_norm_rope_partial(xp, 4 * 64, xp + 512, xp + 1024, 2 * 64, gp, gp, 4, &kv, pos.data(), 1e4, 1e-6f, 0,
                                32, kc.data(), vc.data(), nullptr),
           Q4_ERR_HIP);
    size_t aws = gqa_decode_attn_workspace(&kv, 4, 0);
    std::vector<uint8_t> awv(aws + 512);
    void *aw = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(awv.data()) + 255) / 256 * 256);
    expect_rejected("attn 3 q heads over 2 kv", gqa_decode_attn(xp, 3 * 64, 3, kc.data(), vc.data(), &kv, pos.data(),
                                                                0, 0.125f, yp, 3 * 64, aw, aws, nullptr));
    expect_rejected("attn small ws", gqa_decode_attn(xp, 4 * 64, 4, kc.data(), vc.data(), &kv, pos.data(), 0, 0.125f,
                                                     yp, 4 * 64, aw, 0, nullptr));
    expect("attn valid", gqa_decode_attn(xp, 4 * 64, 4, kc.data(), vc.data(), &kv, pos.data(), 0, 0.125f, yp, 4 * 64,
                                         aw, aws, nullptr),
           Q4_ERR_HIP);
    expect("attn rope valid", gqa_decode_attn_rope(xp, 8 * 64, 4, gp, gp, &kv, pos.data(), 1e4, 1e-6f, 0, kc.data(),
                                                   vc.data(), 0, 0.125f, yp, 4 * 64, aw, aws, nullptr),
           Q4_ERR_HIP);

    // ---- argmax
    expect_rejected("argmax V=0", argmax_rows(xp, 1, 0, tok.data(), nullptr));
    expect("argmax valid", argmax_rows(xp, 2, 1000, tok.data(), nullptr), Q4_ERR_HIP);
    size_t amw = argmax_rows_workspace(2);
    std::vector<uint8_t> amv(amw + 512);
    void *am = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(amv.data()) + 255) / 256 * 256);
    expect("argmax ws valid", argmax_rows_ws(xp, 2, 100000, tok.data(), am, amw, nullptr), Q4_ERR_HIP);

    // ---- decode model
    const int64_t d = 256, hq = 4, hd = 64, ffn = 512, vocab = 1000, batch = 2;
    std::vector<uint8_t> wq(64 + ((hq + 4) * hd) * (d / 32) * 18), wo(64 + d * (hq * hd / 32) * 18),
        wgu(64 + 2 * ffn * (d / 32) * 18), wd(64 + d * (ffn / 32) * 18), emb(64 + vocab * (d / 32) * 34);
    auto al = [](std::vector<uint8_t> &v) {
        return reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(v.data()) + 63) / 64 * 64);
    };
    std::vector<float> kcache(batch * 2 * 64 * hd + 64), vcache(kcache.size());
    q4_layer_desc L{};
    L.wqkv = al(wq);
    L.wo = al(wo);
    L.wgu = al(wgu);
    L.wd = al(wd);
    L.attn_norm = L.ffn_norm = gp;
    L.q_norm = L.k_norm = gp;
    L.k_cache = kcache.data();
    L.v_cache = vcache.data();
    L.n_kv_heads = 2;
    L.head_dim = hd;
    L.cap = 64;
    L.window = 0;
    L.rope_theta = 1e4;
    L.attn_scale = 0.125f;
    q4_model_desc M{};
    M.n_layers = 1;
    M.d_model = d;
    M.n_q_heads = hq;
    M.ffn = ffn;
    M.vocab = vocab;
    M.batch = batch;
    M.eps = 1e-6f;
    M.embed = al(emb);
    M.final_norm = gp;
    M.layers = &L;
    size_t mws = 0;
    expect("decode workspace", decode_model_workspace(&M, &mws), Q4_OK);
    q4_model_desc Mb = M;
    Mb.batch = 0;
    expect_rejected("decode workspace batch 0", decode_model_workspace(&Mb, &mws));
    expect("decode workspace again", decode_model_workspace(&M, &mws), Q4_OK);
    std::vector<uint8_t> mwv(mws + 512);
    void *mw = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(mwv.data()) + 255) / 256 * 256);
    q4_decode_model *model = nullptr;
    expect_rejected("decode create small ws", decode_model_create(&M, mw, 16, &model));
    expect_rejected("decode create null out", decode_model_create(&M, mw, mws, nullptr));
    q4_status st = decode_model_create(&M, mw, mws, &model);
    expect("decode create valid", st, Q4_ERR_HIP);
    if (st == Q4_OK) decode_model_destroy(model);
    expect_rejected("set position null", decode_model_set_position(nullptr, 0, nullptr));
    expect_rejected("decode step null", decode_step(nullptr, tok.data(), tok.data(), nullptr, nullptr));
    expect_rejected("decode eager null", decode_step_eager(nullptr, tok.data(), tok.data(), nullptr, nullptr));
    decode_model_destroy(nullptr);

    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("C ABI host checks under sanitizers: ok (%s)\n", q4dec_version());
    return 0;
}
