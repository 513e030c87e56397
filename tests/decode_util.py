"""Helpers of the decode-step GPU tests: GPU and oracle greedy loops, and a
step recomposed op by op from the C-ABI calls with every op checked against
the oracle fed the GPU's own inputs (lockstep)."""
import numpy as np

from synth import workloads as wl
from synth.device import model_kwargs, prefilled_caches, upload_model  # noqa: F401 (re-exported)


def gpu_model(q, m, dev_model):
    return q.DecodeModel(**model_kwargs(m, dev_model))


def run_gpu(q, m, dev_model, steps, eager=False, want_logits=True):
    """Greedy loop on the GPU; returns (tokens [steps, B], logits [steps, B, V] or None)."""
    import torch
    dev = dev_model["embed"].device
    dm = gpu_model(q, m, dev_model)
    dm.set_position(m.start_pos)
    tok = torch.from_numpy(wl.start_tokens(m)).to(dev)
    nxt = torch.empty_like(tok)
    logits = torch.empty((m.batch, m.vocab), dtype=torch.float32, device=dev) if want_logits else None
    toks, lgs = [], []
    for _ in range(steps):
        dm.step(tok, nxt, logits, eager=eager)
        toks.append(nxt.cpu().numpy().copy())
        if want_logits:
            lgs.append(logits.cpu().numpy().copy())
        tok.copy_(nxt)
    torch.cuda.synchronize()
    dm.close()
    return np.stack(toks), (np.stack(lgs) if want_logits else None)


def run_oracle(oracle, m, weights, steps, want_logits=True, caches=None):
    """Greedy loop of the oracle; ``caches`` (modified in place) default to the recipe's."""
    if caches is None:
        caches = prefilled_caches(m)
    om = oracle.Model(wl.oracle_spec(m, weights, caches))
    tok = wl.start_tokens(m)
    toks, lgs, margins = [], [], []
    for s in range(steps):
        nxt, lg, mg = om.step(m.start_pos + s, tok, want_logits=want_logits)
        toks.append(nxt.copy())
        margins.append(mg.copy())
        if want_logits:
            lgs.append(lg)
        tok = nxt
    return np.stack(toks), (np.stack(lgs) if want_logits else None), np.stack(margins)


def check(got, ref, tol, what, report=None):
    """max |got - ref| / tol <= 1 elementwise; returns the ratio."""
    if hasattr(got, "detach"):
        got = got.detach().cpu().numpy()
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    ratio = float((np.abs(got - ref) / tol).max())
    if report is not None:
        report[what] = ratio
    assert ratio <= 1.0, f"{what}: max err/tol {ratio:.3e}"
    return ratio


def lockstep_step(q, oracle, m, weights, dmod, dev, say=print, caches_ids=None):
    """Recomposes one decode step of model ``m`` (uploaded as ``dmod``, host
    weights ``weights``) from the C-ABI calls the library's step makes, in its
    order, and checks each call's output against the oracle op fed the GPU's
    own inputs.  Returns (next tokens, logits) as device tensors and a dict of
    the worst err/tol per op.  The plain pre-norm block only (no sandwich
    norms, no p-RoPE)."""
    import torch
    from q4_quantized_matvec_amd._lib import kv_layout_of

    B, D, Hq, F, eps = m.batch, m.d_model, m.n_q_heads, m.ffn, m.eps
    pos = m.start_pos
    tok = torch.from_numpy(wl.start_tokens(m)).to(dev)
    rep = {}
    np_ = lambda t: t.detach().cpu().numpy().astype(np.float64)

    def proj(fmt, W, xx, K, ld, op, **kw):
        # the step runs its projections on the matrix cores when B >= 2
        if B >= 2 and K % 256 == 0:
            fn = q.q4_0_matvec_batched if fmt == 4 else q.q8_0_matvec_batched
        else:
            fn = q.q4_0_matvec_fused if fmt == 4 else q.q8_0_matvec_fused
        return fn(W, xx, K, B, ld, op, eps=eps, **kw)

    pos_d = torch.tensor([pos, pos + 1], dtype=torch.int64, device=dev)
    x = q.q8_0_gather(dmod["embed"], tok, D)
    check(x, oracle.q8_0_gather(weights["embed"], m.vocab, D, tok.cpu().numpy()),
          np.full((B, D), 1e-30), "gather (exact)", rep)
    for l, ly in enumerate(m.layers):
        assert ly.rope_dims == 0 and not m.sandwich and m.ffn_act == "silu"
        L, W = dmod["layers"][l], weights["layers"][l]
        hd, hkv = ly.head_dim, ly.n_kv_heads
        nq, nk, nv = wl.layer_rows(m, ly)
        nqkv = nq + nk + nv
        say(f"  lockstep layer {l}: hd {hd}, {hkv} kv heads, window {ly.window}, cap {ly.cap}")
        qkv = proj(4, L["wqkv"], x, D, D, q.IN_RMSNORM, norm_w=L["attn_norm"])
        r, t = oracle.q4_0_matvec(W["wqkv"], nqkv, D, oracle.rmsnorm(np_(x), W["attn_norm"], eps))
        check(qkv, r, 2e-4 * t + 1e-6, f"L{l} rmsnorm + qkv matvec", rep)
        raw = np_(qkv).copy()
        kv = kv_layout_of(L["k_cache"])
        ws = torch.zeros(q.gqa_decode_attn_workspace(kv, Hq, ly.window), dtype=torch.uint8, device=dev)
        att = torch.empty((B, nq), dtype=torch.float32, device=dev)
        # the step fuses QK-norm, RoPE and the KV append into the attention call
        q.gqa_decode_attn_rope(qkv, nqkv, Hq, L["q_norm"], L["k_norm"], kv, pos_d[0:1], ly.rope_theta,
                               eps, ly.v_from_k, L["k_cache"], L["v_cache"], ly.window,
                               ly.attn_scale, att, nq, ws)
        slot = pos % ly.cap
        n = pos + 1
        lo = max(0, n - ly.window) if ly.window else 0
        vis = np.arange(lo, n)
        kc_t, vc_t = L["k_cache"], L["v_cache"]
        for b in range(B):
            kr = raw[b, nq:nq + nk].reshape(hkv, hd)
            kref = oracle.rope_neox(oracle.rmsnorm(kr, W["k_norm"], eps), pos, ly.rope_theta)
            check(np_(kc_t[b, :, slot]), kref, 2e-4 * np.abs(kref) + 2e-5, f"L{l} appended key", rep)
            vref = (oracle.rmsnorm(kr, None, eps) if ly.v_from_k
                    else raw[b, nq + nk:].reshape(hkv, hd))
            check(np_(vc_t[b, :, slot]), vref, 2e-4 * np.abs(vref) + 1e-6, f"L{l} appended value", rep)
            qh = oracle.rope_neox(oracle.rmsnorm(raw[b, :nq].reshape(Hq, hd), W["q_norm"], eps),
                                  pos, ly.rope_theta)
            # the visible positions' rows, read back from their slots (a ring
            # wraps: position p lives in slot p % cap)
            sl = torch.from_numpy(vis % ly.cap).to(dev)
            keys = np.zeros((n, hkv, hd))
            vals = np.zeros((n, hkv, hd))
            keys[lo:] = np_(kc_t[b][:, sl].permute(1, 0, 2))
            vals[lo:] = np_(vc_t[b][:, sl].permute(1, 0, 2))
            o, bound = oracle.gqa_attention(qh, keys, vals, ly.window, ly.attn_scale)
            check(att[b], o, 2e-4 * bound + 1e-6, f"L{l} attention", rep)
        xo = np_(x)
        proj(4, L["wo"], att, nq, nq, q.IN_PLAIN, y=x, residual=x)
        r, t = oracle.q4_0_matvec(W["wo"], D, nq, np_(att), res=xo)
        check(x, r, 2e-4 * t + 1e-6, f"L{l} o-proj + residual", rep)
        # the step hands SiLU(gate) * up from the gate|up kernel to the down projection
        h = proj(4, L["wgu"], x, D, D, q.IN_RMSNORM, norm_w=L["ffn_norm"], out_op=q.OUT_SWIGLU)
        r, t = oracle.q4_0_matvec(W["wgu"], 2 * F, D, oracle.rmsnorm(np_(x), W["ffn_norm"], eps))
        g, u = r[:, :F], r[:, F:]
        tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
        h_ref = np.stack([oracle.swiglu(g[b], u[b]) for b in range(B)])
        silu_g = g / (1.0 + np.exp(-g))
        check(h, h_ref, 1.1 * tg * np.abs(u) + np.abs(silu_g) * tu + 2e-4 * np.abs(h_ref) + 1e-6,
              f"L{l} rmsnorm + gate|up + swiglu", rep)
        xo = np_(x)
        proj(4, L["wd"], h, F, F, q.IN_PLAIN, y=x, residual=x)
        r, t = oracle.q4_0_matvec(W["wd"], D, F, np_(h), res=xo)
        check(x, r, 2e-4 * t + 1e-6, f"L{l} down + residual", rep)
    logits = proj(8, dmod["embed"], x, D, D, q.IN_RMSNORM, norm_w=dmod["final_norm"])
    r, t = oracle.q8_0_matvec(weights["embed"], m.vocab, D,
                              oracle.rmsnorm(np_(x), weights["final_norm"], eps))
    check(logits, r, 2e-4 * t + 1e-6, "final rmsnorm + logits", rep)
    nxt = q.argmax_rows(logits)
    lg = np_(logits)
    assert nxt.cpu().numpy().tolist() == [oracle.argmax(lg[b])[0] for b in range(B)]
    return tok, nxt, logits, rep


def _gated_ref(oracle, r, t, F, act):
    """Reference and bound of a gated output (gate rows, then up rows of r)."""
    g, u = r[:, :F], r[:, F:]
    tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
    fn = oracle.geglu if act == "gelu_tanh" else oracle.swiglu
    ref = np.stack([fn(g[b], u[b]) for b in range(r.shape[0])])
    tol = 1.13 * tg * np.abs(u) + np.abs(np.stack([fn(g[b], np.ones_like(g[b])) for b in range(r.shape[0])])) \
        * tu + 2e-4 * np.abs(ref) + 1e-6
    return ref, tol


def lockstep_step_variants(q, oracle, m, weights, dmod, dev, say=print):
    """As lockstep_step for a model with the Gemma-4 block variants at B = 1
    (where the library's step takes the vector kernels): the scaled embedding
    gather; sandwich post-norms, each joining the residual stream inside the
    next pre-normed projection (q4_0_matvec_post_norm, the stream alternating
    between two buffers) and the last one by rmsnorm_add; p-RoPE layers
    prepared by qk_norm_rope_partial and attended by gqa_decode_attn; GeGLU
    or SwiGLU output of gate|up; the soft-capped logits.  Every call is
    checked against the oracle fed the GPU's own inputs.  Returns (tokens,
    next tokens, logits, worst err/tol per op)."""
    import torch
    from q4_quantized_matvec_amd._lib import kv_layout_of

    B, D, Hq, F, eps = m.batch, m.d_model, m.n_q_heads, m.ffn, m.eps
    assert B == 1 and D % 256 == 0 and D <= 8192, "the vector-kernel form of the step"
    pos = m.start_pos
    tok = torch.from_numpy(wl.start_tokens(m)).to(dev)
    rep = {}
    np_ = lambda t: t.detach().cpu().numpy().astype(np.float64)
    gout = q.OUT_GEGLU if m.ffn_act == "gelu_tanh" else q.OUT_SWIGLU
    pos_d = torch.tensor([pos, pos + 1], dtype=torch.int64, device=dev)

    scale = float(np.float32(m.embed_scale)) if m.embed_scale and m.embed_scale != 1.0 else None
    hc = q.q8_0_gather(dmod["embed"], tok, D, scale=scale)
    ref = oracle.q8_0_gather(weights["embed"], m.vocab, D, tok.cpu().numpy()) * (scale or 1.0)
    # one fp32 rounding of the exact (d q) s: at most half an ulp of the result
    check(hc, ref, 2.0 ** -24 * (1.0 + 2.0 ** -20) * np.abs(ref) + 1e-30, "gather (scaled)", rep)
    ha = torch.empty_like(hc)
    tmp = torch.empty_like(hc)
    pend = None  # (device gain, host gain) of a post-norm waiting in tmp

    def normed_proj(Wd, Wh, N, gd, gh, out_op, what):
        nonlocal hc, ha, pend
        if pend is not None:
            pwd, pwh = pend
            y = q.q4_0_matvec_post_norm(Wd, hc, tmp, D, B, D, pwd, gd, eps, ha, n=N, out_op=out_op)
            normed = oracle.rmsnorm(np_(tmp), pwh, eps)
            ref_h = np_(hc) + normed
            check(ha, ref_h, 2e-4 * np.abs(normed) + 2.0 ** -23 * np.abs(ref_h) + 1e-6,
                  f"{what}: post-norm joins the stream", rep)
            xin = oracle.rmsnorm(np_(ha), gh, eps)
            hc, ha = ha, hc
            pend = None
        else:
            y = q.q4_0_matvec_fused(Wd, hc, D, B, D, q.IN_RMSNORM, norm_w=gd, eps=eps, n=N, out_op=out_op)
            xin = oracle.rmsnorm(np_(hc), gh, eps)
        r, t = oracle.q4_0_matvec(Wh, N, D, xin)
        if out_op == q.OUT_PLAIN:
            check(y, r, 2e-4 * t + 1e-6, f"{what}: rmsnorm + matvec", rep)
        else:
            gref, gtol = _gated_ref(oracle, r, t, N // 2, m.ffn_act)
            check(y, gref, gtol, f"{what}: rmsnorm + matvec + gated output", rep)
        return y

    for l, ly in enumerate(m.layers):
        L, W = dmod["layers"][l], weights["layers"][l]
        hd, hkv = ly.head_dim, ly.n_kv_heads
        nq, nk, nv = wl.layer_rows(m, ly)
        nqkv = nq + nk + nv
        say(f"  lockstep layer {l}: hd {hd}, {hkv} kv heads, window {ly.window}, cap {ly.cap}, "
            f"rotated dims {ly.rope_dims or hd}")
        qkv = normed_proj(L["wqkv"], W["wqkv"], nqkv, L["attn_norm"], W["attn_norm"], q.OUT_PLAIN, f"L{l} qkv")
        raw = np_(qkv).copy()
        kv = kv_layout_of(L["k_cache"])
        ws = torch.zeros(q.gqa_decode_attn_workspace(kv, Hq, ly.window), dtype=torch.uint8, device=dev)
        att = torch.empty((B, nq), dtype=torch.float32, device=dev)
        rot = ly.rope_dims if ly.rope_dims else hd
        partial = rot != hd
        if partial:
            q.qk_norm_rope(qkv, nqkv, qkv[:, nq:], None if ly.v_from_k else qkv[:, nq + nk:], nqkv,
                           L["q_norm"], L["k_norm"], Hq, kv, pos_d[0:1], ly.rope_theta, eps, ly.v_from_k,
                           L["k_cache"], L["v_cache"], rot_dims=rot)
            q.gqa_decode_attn(qkv, nqkv, Hq, L["k_cache"], L["v_cache"], kv, pos_d[1:2], ly.window,
                              ly.attn_scale, att, nq, ws)
        else:
            q.gqa_decode_attn_rope(qkv, nqkv, Hq, L["q_norm"], L["k_norm"], kv, pos_d[0:1], ly.rope_theta,
                                   eps, ly.v_from_k, L["k_cache"], L["v_cache"], ly.window,
                                   ly.attn_scale, att, nq, ws)
        slot = pos % ly.cap
        n = pos + 1
        lo = max(0, n - ly.window) if ly.window else 0
        vis = np.arange(lo, n)
        kc_t, vc_t = L["k_cache"], L["v_cache"]
        for b in range(B):
            kr = raw[b, nq:nq + nk].reshape(hkv, hd)
            kref = oracle.rope_neox(oracle.rmsnorm(kr, W["k_norm"], eps), pos, ly.rope_theta,
                                    rot if partial else 0)
            check(np_(kc_t[b, :, slot]), kref, 2e-4 * np.abs(kref) + 2e-5, f"L{l} appended key", rep)
            vref = (oracle.rmsnorm(kr, None, eps) if ly.v_from_k
                    else raw[b, nq + nk:].reshape(hkv, hd))
            check(np_(vc_t[b, :, slot]), vref, 2e-4 * np.abs(vref) + 1e-6, f"L{l} appended value", rep)
            qh = oracle.rope_neox(oracle.rmsnorm(raw[b, :nq].reshape(Hq, hd), W["q_norm"], eps),
                                  pos, ly.rope_theta, rot if partial else 0)
            if partial:  # the prepared query is written back in place; attention reads it
                check(np_(qkv[b, :nq]).reshape(Hq, hd), qh, 2e-4 * np.abs(qh) + 2e-5,
                      f"L{l} p-RoPE query", rep)
                qh = np_(qkv[b, :nq]).reshape(Hq, hd)
            sl = torch.from_numpy(vis % ly.cap).to(dev)
            keys = np.zeros((n, hkv, hd))
            vals = np.zeros((n, hkv, hd))
            keys[lo:] = np_(kc_t[b][:, sl].permute(1, 0, 2))
            vals[lo:] = np_(vc_t[b][:, sl].permute(1, 0, 2))
            o, bound = oracle.gqa_attention(qh, keys, vals, ly.window, ly.attn_scale)
            check(att[b], o, 2e-4 * bound + 1e-6, f"L{l} attention", rep)
        # O projection: with a post-norm its output waits in tmp
        if W.get("post_attn_norm") is not None:
            q.q4_0_matvec_fused(L["wo"], att, nq, B, nq, q.IN_PLAIN, y=tmp)
            r, t = oracle.q4_0_matvec(W["wo"], D, nq, np_(att))
            check(tmp, r, 2e-4 * t + 1e-6, f"L{l} o-proj", rep)
            pend = (L["post_attn_norm"], W["post_attn_norm"])
        else:
            xo = np_(hc)
            q.q4_0_matvec_fused(L["wo"], att, nq, B, nq, q.IN_PLAIN, y=hc, residual=hc)
            r, t = oracle.q4_0_matvec(W["wo"], D, nq, np_(att), res=xo)
            check(hc, r, 2e-4 * t + 1e-6, f"L{l} o-proj + residual", rep)
        h = normed_proj(L["wgu"], W["wgu"], 2 * F, L["ffn_norm"], W["ffn_norm"], gout, f"L{l} gate|up")
        if W.get("post_ffn_norm") is not None:
            q.q4_0_matvec_fused(L["wd"], h, F, B, F, q.IN_PLAIN, y=tmp)
            r, t = oracle.q4_0_matvec(W["wd"], D, F, np_(h))
            check(tmp, r, 2e-4 * t + 1e-6, f"L{l} down", rep)
            pend = (L["post_ffn_norm"], W["post_ffn_norm"])
        else:
            xo = np_(hc)
            q.q4_0_matvec_fused(L["wd"], h, F, B, F, q.IN_PLAIN, y=hc, residual=hc)
            r, t = oracle.q4_0_matvec(W["wd"], D, F, np_(h), res=xo)
            check(hc, r, 2e-4 * t + 1e-6, f"L{l} down + residual", rep)
    if pend is not None:
        x0 = np_(hc)
        q.rmsnorm_add(tmp, pend[0], eps, hc)
        normed = oracle.rmsnorm(np_(tmp), pend[1], eps)
        ref_h = x0 + normed
        check(hc, ref_h, 2e-4 * np.abs(normed) + 2.0 ** -23 * np.abs(ref_h) + 1e-6,
              "last post-norm (rmsnorm_add)", rep)
    logits = q.q8_0_matvec_fused(dmod["embed"], hc, D, B, D, q.IN_RMSNORM, norm_w=dmod["final_norm"], eps=eps)
    r, t = oracle.q8_0_matvec(weights["embed"], m.vocab, D, oracle.rmsnorm(np_(hc), weights["final_norm"], eps))
    check(logits, r, 2e-4 * t + 1e-6, "final rmsnorm + logits", rep)
    if m.logit_softcap:
        before = np_(logits)
        q.softcap(logits, m.logit_softcap)
        check(logits, oracle.softcap(before, m.logit_softcap), np.full(before.shape, 2e-6 * m.logit_softcap),
              "soft cap", rep)
    nxt = q.argmax_rows(logits)
    lg = np_(logits)
    assert nxt.cpu().numpy().tolist() == [oracle.argmax(lg[b])[0] for b in range(B)]
    return tok, nxt, logits, rep
