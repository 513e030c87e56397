"""Oracle decode step: invariants of the composition of the pinned parts.

The whole-step result itself is parity-unpinned beyond these properties (the
pages print no worked decode example for synthetic weights).
"""
import numpy as np
import pytest

import oracle
from synth import workloads as wl


def _fresh(m, weights):
    caches = [(wl.prefilled_cache(m, l, "k"), wl.prefilled_cache(m, l, "v"))
              for l in range(m.n_layers)]
    return oracle.Model(wl.oracle_spec(m, weights, caches)), caches


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4], ids=lambda s: s.name)
def test_decode_deterministic(shape):
    w = wl.model_weights(shape)
    tok = wl.start_tokens(shape)
    outs = []
    for _ in range(2):
        model, _ = _fresh(shape, w)
        nxt, logits, _ = model.step(shape.start_pos, tok, want_logits=True)
        outs.append((nxt, logits))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_decode_independent_of_thread_count():
    """Threads split independent outputs only, so one thread and all threads
    give the same step bit for bit (the CPU baseline times both)."""
    shape = wl.TINY_GEMMA4
    w = wl.model_weights(shape)
    tok = wl.start_tokens(shape)
    full = oracle.num_threads()
    outs = []
    try:
        for n in (1, full):
            oracle.set_num_threads(n)
            assert oracle.num_threads() == n
            model, _ = _fresh(shape, w)
            outs.append(model.step(shape.start_pos, tok, want_logits=True)[:2])
    finally:
        oracle.set_num_threads(full)
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4], ids=lambda s: s.name)
def test_decode_batch_rows_independent(shape):
    """A batch of B sequences equals B separate single-sequence steps, bit for bit."""
    w = wl.model_weights(shape)
    tok = wl.start_tokens(shape)
    model, caches = _fresh(shape, w)
    nxt, logits, _ = model.step(shape.start_pos, tok, want_logits=True)
    one = wl.replace(shape, batch=1)
    for b in range(shape.batch):
        cb = [(np.ascontiguousarray(k[b:b + 1]), np.ascontiguousarray(v[b:b + 1]))
              for (k, v) in [(wl.prefilled_cache(shape, l, "k"), wl.prefilled_cache(shape, l, "v"))
                             for l in range(shape.n_layers)]]
        m1 = oracle.Model(wl.oracle_spec(one, w, cb))
        n1, l1, _ = m1.step(shape.start_pos, tok[b:b + 1], want_logits=True)
        assert n1[0] == nxt[b]
        assert np.array_equal(l1[0], logits[b])
        for l in range(shape.n_layers):
            assert np.array_equal(cb[l][0][0], caches[l][0][b])
            assert np.array_equal(cb[l][1][0], caches[l][1][b])


def test_decode_identical_sequences_give_identical_rows():
    shape = wl.TINY_QWEN3
    w = wl.model_weights(shape)
    caches = []
    for l in range(shape.n_layers):
        k = wl.prefilled_cache(shape, l, "k")
        v = wl.prefilled_cache(shape, l, "v")
        k[:] = k[0:1]
        v[:] = v[0:1]
        caches.append((k, v))
    model = oracle.Model(wl.oracle_spec(shape, w, caches))
    tok = np.full(shape.batch, 17, dtype=np.int32)
    nxt, logits, _ = model.step(shape.start_pos, tok, want_logits=True)
    assert np.all(nxt == nxt[0])
    for b in range(1, shape.batch):
        assert np.array_equal(logits[b], logits[0])


def _compose_one_step(shape, w, caches, pos, tok):
    """The block topology restated with the separately pinned oracle ops."""
    B, D, Hq, F = shape.batch, shape.d_model, shape.n_q_heads, shape.ffn
    x = oracle.q8_0_gather(w["embed"], shape.vocab, D, tok)
    if shape.embed_scale:
        x = x * shape.embed_scale
    for l, ly in enumerate(shape.layers):
        L = w["layers"][l]
        hd, hkv = ly.head_dim, ly.n_kv_heads
        nq, nk, nv = wl.layer_rows(shape, ly)
        xn = oracle.rmsnorm(x, L["attn_norm"], shape.eps)
        qkv, _ = oracle.q4_0_matvec(L["wqkv"], nq + nk + nv, D, xn)
        att = np.empty((B, nq))
        for b in range(B):
            q = qkv[b, :nq].reshape(Hq, hd)
            kr = qkv[b, nq:nq + nk].reshape(hkv, hd)
            v = (oracle.rmsnorm(kr, None, shape.eps) if ly.v_from_k
                 else qkv[b, nq + nk:].reshape(hkv, hd))
            q = oracle.rope_neox(oracle.rmsnorm(q, L["q_norm"], shape.eps), pos, ly.rope_theta,
                                 ly.rope_dims)
            k = oracle.rope_neox(oracle.rmsnorm(kr, L["k_norm"], shape.eps), pos, ly.rope_theta,
                                 ly.rope_dims)
            kc, vc = caches[l]
            kc[b, :, pos % ly.cap] = k.astype(np.float32)
            vc[b, :, pos % ly.cap] = v.astype(np.float32)
            n = pos + 1
            lo = max(0, n - ly.window) if ly.window else 0
            slots = [p % ly.cap for p in range(n)]
            keys = np.zeros((n, hkv, hd))
            vals = np.zeros((n, hkv, hd))
            for p in range(lo, n):
                keys[p] = kc[b, :, slots[p]]
                vals[p] = vc[b, :, slots[p]]
            o, _ = oracle.gqa_attention(q, keys, vals, ly.window, ly.attn_scale)
            att[b] = o.reshape(-1)
        if shape.sandwich:
            o_, _ = oracle.q4_0_matvec(L["wo"], D, nq, att)
            x = x + oracle.rmsnorm(o_, L["post_attn_norm"], shape.eps)
        else:
            x, _ = oracle.q4_0_matvec(L["wo"], D, nq, att, res=x)
        xn = oracle.rmsnorm(x, L["ffn_norm"], shape.eps)
        gu, _ = oracle.q4_0_matvec(L["wgu"], 2 * F, D, xn)
        act = oracle.geglu if shape.ffn_act == "gelu_tanh" else oracle.swiglu
        h = act(gu[:, :F], gu[:, F:])
        if shape.sandwich:
            d_, _ = oracle.q4_0_matvec(L["wd"], D, F, h)
            x = x + oracle.rmsnorm(d_, L["post_ffn_norm"], shape.eps)
        else:
            x, _ = oracle.q4_0_matvec(L["wd"], D, F, h, res=x)
    xn = oracle.rmsnorm(x, w["final_norm"], shape.eps)
    logits, _ = oracle.q8_0_matvec(w["embed"], shape.vocab, D, xn)
    if shape.logit_softcap:
        logits = oracle.softcap(logits, shape.logit_softcap)
    return logits


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4, wl.TINY_GEMMA4_EXACT,
                                   wl.TINY_GEMMA4_EXACT_B1],
                         ids=lambda s: s.name)
def test_decode_equals_composition_of_pinned_ops(shape):
    w = wl.model_weights(shape)
    tok = wl.start_tokens(shape)
    model, caches = _fresh(shape, w)
    pos = shape.start_pos
    for step in range(2):
        comp_caches = [(k.copy(), v.copy()) for (k, v) in caches]
        ref = _compose_one_step(shape, w, comp_caches, pos, tok)
        nxt, logits, margins = model.step(pos, tok, want_logits=True)
        assert np.allclose(logits, ref, rtol=1e-12, atol=1e-12)
        assert np.array_equal(nxt, ref.argmax(axis=1))
        assert np.all(margins >= 0)
        for l in range(shape.n_layers):
            assert np.array_equal(comp_caches[l][0], caches[l][0])
        tok = nxt
        pos += 1


def test_gemma_exact_variants_change_the_step():
    """Each Gemma-4 variant is live: switching any one of them off changes the
    logits (the soft cap alone leaves the tokens unchanged: tanh is
    increasing)."""
    import dataclasses
    m = wl.TINY_GEMMA4_EXACT
    w = wl.model_weights(m)
    tok = wl.start_tokens(m)

    def run(shape):
        caches = [(wl.prefilled_cache(shape, l, "k"), wl.prefilled_cache(shape, l, "v"))
                  for l in range(shape.n_layers)]
        spec = wl.oracle_spec(shape, w, caches)
        if not shape.sandwich:
            for L in spec["layers"]:
                L["post_attn_norm"] = L["post_ffn_norm"] = None
        return oracle.Model(spec).step(shape.start_pos, tok, want_logits=True)

    n0, l0, _ = run(m)
    no_cap = dataclasses.replace(m, logit_softcap=0.0)
    n1, l1, _ = run(no_cap)
    assert np.array_equal(n0, n1)
    assert np.allclose(l0, oracle.softcap(l1, m.logit_softcap), rtol=1e-13, atol=1e-13)
    full_rope = dataclasses.replace(
        m, layers=tuple(dataclasses.replace(ly, rope_dims=0) for ly in m.layers))
    for variant in (dataclasses.replace(m, ffn_act="silu"), dataclasses.replace(m, embed_scale=0.0),
                    dataclasses.replace(m, sandwich=False), full_rope):
        _, lv, _ = run(variant)
        assert np.abs(lv - l0).max() > 1e-6
