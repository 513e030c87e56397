"""GPU decode step (HIP graph) against the fp64 oracle.

Per-op parity is checked in lockstep: the step is recomposed from the same
C-ABI calls, each call's output is compared with the oracle op fed the GPU's
own inputs, and the composition is checked to equal the library's step bit
for bit.  End to end, the greedy tokens must be identical to the oracle's at
every step; the logit NMSE and top-2 margins are reported.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
from q4_quantized_matvec_amd._lib import kv_layout_of
from synth import workloads as wl

from decode_util import gpu_model, prefilled_caches, run_gpu, run_oracle, upload_model

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _nmse(a, b):
    return float(((a - b) ** 2).sum() / (b ** 2).sum())


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4, wl.TINY_GEMMA4_LONG,
                                   wl.TINY_QWEN3_B20, wl.TINY_GEMMA4_EXACT,
                                   wl.TINY_GEMMA4_EXACT_B1], ids=lambda s: s.name)
def test_decode_tokens_match_oracle(dev, shape):
    _say(f"decode {shape.name}: {shape.steps} steps")
    weights = wl.model_weights(shape)
    toks_o, lg_o, margins = run_oracle(oracle, shape, weights, shape.steps)
    toks_g, lg_g = run_gpu(q, shape, upload_model(shape, weights, dev), shape.steps)
    nmse = _nmse(lg_g.astype(np.float64), lg_o)
    _say(f"  tokens gpu {toks_g.tolist()} oracle {toks_o.tolist()} nmse {nmse:.3e} "
         f"min margin {margins.min():.4f}")
    assert np.array_equal(toks_g, toks_o)
    assert nmse < 1e-8


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4, wl.TINY_GEMMA4_LONG],
                         ids=lambda s: s.name)
def test_decode_f16_kv_matches_oracle(dev, shape):
    """Binary16 KV caches on both sides (the same prefilled values; each side
    appends its rows rounded to the nearest binary16).  Where the GPU's fp32
    row and the oracle's fp64 row fall on the two sides of a rounding
    midpoint the appended elements differ by one unit in the last place
    (2^-10 relative), and that difference carries through later steps; so
    besides identical tokens the logits must be much closer to the oracle's
    binary16 decode than binary16 caching itself moves them (the oracle's
    binary16 decode against its fp32 one)."""
    _say(f"decode {shape.name} with binary16 caches: {shape.steps} steps")
    weights = wl.model_weights(shape)
    orc_caches = prefilled_caches(shape, kv16=True)
    toks_o, lg_o, margins = run_oracle(oracle, shape, weights, shape.steps, caches=orc_caches)
    _, lg_o32, _ = run_oracle(oracle, shape, weights, shape.steps)
    dmod = upload_model(shape, weights, dev, caches=prefilled_caches(shape, kv16=True))
    assert all(L["k_cache"].dtype == torch.float16 for L in dmod["layers"])
    toks_g, lg_g = run_gpu(q, shape, dmod, shape.steps)
    nmse = _nmse(lg_g.astype(np.float64), lg_o)
    effect = _nmse(lg_o, lg_o32)
    # layer 0 of the first step sees the same inputs on both sides: its
    # appended elements agree to one unit in the last place
    ly0 = shape.layers[0]
    slot = shape.start_pos % ly0.cap
    ulps = []
    for c, key in enumerate(("k_cache", "v_cache")):
        g16 = dmod["layers"][0][key][:, :, slot].cpu().numpy().view(np.uint16).astype(np.int64)
        o16 = orc_caches[0][c][:, :, slot].view(np.uint16).astype(np.int64)
        ulps.append(int(np.abs(g16 - o16).max()))
    _say(f"  tokens gpu {toks_g.tolist()} oracle {toks_o.tolist()} nmse {nmse:.3e} "
         f"(binary16 caching itself: {effect:.3e}) min margin {margins.min():.4f}; "
         f"layer 0 first appended rows differ by <= {max(ulps)} ulp")
    assert max(ulps) <= 1
    assert np.array_equal(toks_g, toks_o)
    assert nmse < 0.1 * effect


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4, wl.TINY_GEMMA4_LONG,
                                   wl.TINY_QWEN3_B20, wl.TINY_GEMMA4_EXACT,
                                   wl.TINY_GEMMA4_EXACT_B1], ids=lambda s: s.name)
def test_graph_equals_eager(dev, shape):
    _say(f"graph vs eager {shape.name}")
    weights = wl.model_weights(shape)
    dm1 = upload_model(shape, weights, dev)
    t1, l1 = run_gpu(q, shape, dm1, shape.steps, eager=False)
    dm2 = upload_model(shape, weights, dev)
    t2, l2 = run_gpu(q, shape, dm2, shape.steps, eager=True)
    assert np.array_equal(t1, t2) and np.array_equal(l1, l2)
    for a, b in zip(dm1["layers"], dm2["layers"]):
        assert torch.equal(a["k_cache"], b["k_cache"]) and torch.equal(a["v_cache"], b["v_cache"])


def _check(got, ref, tol, what):
    if hasattr(got, "detach"):
        got = got.detach().cpu().numpy()
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    ratio = float((np.abs(got - ref) / tol).max())
    assert ratio <= 1.0, f"{what}: max err/tol {ratio:.3e}"
    return ratio


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4], ids=lambda s: s.name)
def test_decode_lockstep_per_op(dev, shape):
    """Recompose one step from the C-ABI ops; check every op against the oracle
    fed the GPU's inputs, then check the composition equals decode_step_eager."""
    _say(f"lockstep {shape.name}")
    m = shape
    weights = wl.model_weights(m)
    dmod = upload_model(m, weights, dev)
    B, D, Hq, F, eps = m.batch, m.d_model, m.n_q_heads, m.ffn, m.eps
    pos = m.start_pos
    tok = torch.from_numpy(wl.start_tokens(m)).to(dev)

    def proj(fmt, W, xx, K, ld, op, **kw):
        # the step runs its projections on the matrix cores when B >= 2
        if B >= 2 and K % 256 == 0:
            fn = q.q4_0_matvec_batched if fmt == 4 else q.q8_0_matvec_batched
        else:
            fn = q.q4_0_matvec_fused if fmt == 4 else q.q8_0_matvec_fused
        return fn(W, xx, K, B, ld, op, eps=eps, **kw)

    pos_d = torch.tensor([pos, pos + 1], dtype=torch.int64, device=dev)
    x = q.q8_0_gather(dmod["embed"], tok, D)
    _check(x, oracle.q8_0_gather(weights["embed"], m.vocab, D, tok.cpu().numpy()),
           np.full((B, D), 1e-30), "gather (exact)")
    np_ = lambda t: t.detach().cpu().numpy().astype(np.float64)
    for l, ly in enumerate(m.layers):
        L, W = dmod["layers"][l], weights["layers"][l]
        hd, hkv = ly.head_dim, ly.n_kv_heads
        nq, nk, nv = wl.layer_rows(m, ly)
        nqkv = nq + nk + nv
        qkv = proj(4, L["wqkv"], x, D, D, q.IN_RMSNORM, norm_w=L["attn_norm"])
        r, t = oracle.q4_0_matvec(W["wqkv"], nqkv, D, oracle.rmsnorm(np_(x), W["attn_norm"], eps))
        _check(qkv, r, 2e-4 * t + 1e-6, f"L{l} rmsnorm + qkv matvec")
        raw = np_(qkv).copy()
        kv = kv_layout_of(L["k_cache"])
        ws = torch.empty(q.gqa_decode_attn_workspace(kv, Hq, ly.window), dtype=torch.uint8, device=dev)
        att = torch.empty((B, nq), dtype=torch.float32, device=dev)
        # the step fuses QK-norm, RoPE and the KV append into the attention call
        q.gqa_decode_attn_rope(qkv, nqkv, Hq, L["q_norm"], L["k_norm"], kv, pos_d[0:1], ly.rope_theta,
                               eps, ly.v_from_k, L["k_cache"], L["v_cache"], ly.window,
                               ly.attn_scale, att, nq, ws)
        kc, vc = np_(L["k_cache"]), np_(L["v_cache"])
        slot = pos % ly.cap
        for b in range(B):
            kr = raw[b, nq:nq + nk].reshape(hkv, hd)
            kref = oracle.rope_neox(oracle.rmsnorm(kr, W["k_norm"], eps), pos, ly.rope_theta)
            _check(kc[b, :, slot], kref, 2e-4 * np.abs(kref) + 2e-5, f"L{l} appended key")
            vref = (oracle.rmsnorm(kr, None, eps) if ly.v_from_k
                    else raw[b, nq + nk:].reshape(hkv, hd))
            _check(vc[b, :, slot], vref, 2e-4 * np.abs(vref) + 1e-6, f"L{l} appended value")
            qh = oracle.rope_neox(oracle.rmsnorm(raw[b, :nq].reshape(Hq, hd), W["q_norm"], eps),
                                  pos, ly.rope_theta)
            n = pos + 1
            lo = max(0, n - ly.window) if ly.window else 0
            keys = np.zeros((n, hkv, hd))
            vals = np.zeros((n, hkv, hd))
            for p in range(lo, n):
                keys[p] = kc[b, :, p % ly.cap]
                vals[p] = vc[b, :, p % ly.cap]
            o, bound = oracle.gqa_attention(qh, keys, vals, ly.window, ly.attn_scale)
            _check(att[b], o, 2e-4 * bound + 1e-6, f"L{l} attention")
        xo = np_(x)
        proj(4, L["wo"], att, nq, nq, q.IN_PLAIN, y=x, residual=x)
        r, t = oracle.q4_0_matvec(W["wo"], D, nq, np_(att), res=xo)
        _check(x, r, 2e-4 * t + 1e-6, f"L{l} o-proj + residual")
        # the step hands SiLU(gate) * up from the gate|up kernel to the down projection
        h = proj(4, L["wgu"], x, D, D, q.IN_RMSNORM, norm_w=L["ffn_norm"], out_op=q.OUT_SWIGLU)
        r, t = oracle.q4_0_matvec(W["wgu"], 2 * F, D, oracle.rmsnorm(np_(x), W["ffn_norm"], eps))
        g, u = r[:, :F], r[:, F:]
        tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
        h_ref = np.stack([oracle.swiglu(g[b], u[b]) for b in range(B)])
        silu_g = g / (1.0 + np.exp(-g))
        _check(h, h_ref, 1.1 * tg * np.abs(u) + np.abs(silu_g) * tu + 2e-4 * np.abs(h_ref) + 1e-6,
               f"L{l} rmsnorm + gate|up + swiglu")
        xo = np_(x)
        proj(4, L["wd"], h, F, F, q.IN_PLAIN, y=x, residual=x)
        r, t = oracle.q4_0_matvec(W["wd"], D, F, np_(h), res=xo)
        _check(x, r, 2e-4 * t + 1e-6, f"L{l} down + residual")
    logits = proj(8, dmod["embed"], x, D, D, q.IN_RMSNORM, norm_w=dmod["final_norm"])
    r, t = oracle.q8_0_matvec(weights["embed"], m.vocab, D,
                              oracle.rmsnorm(np_(x), weights["final_norm"], eps))
    _check(logits, r, 2e-4 * t + 1e-6, "final rmsnorm + logits")
    nxt = q.argmax_rows(logits)
    assert nxt.cpu().numpy().tolist() == [oracle.argmax(np_(logits)[b])[0] for b in range(B)]

    # the library's own step runs the same kernels in the same order: bit-identical
    fresh = upload_model(m, weights, dev)
    dm = gpu_model(q, m, fresh)
    dm.set_position(pos)
    nxt2 = torch.empty_like(tok)
    lg2 = torch.empty((B, m.vocab), dtype=torch.float32, device=dev)
    dm.step(tok, nxt2, lg2, eager=True)
    torch.cuda.synchronize()
    assert torch.equal(lg2, logits) and torch.equal(nxt2, nxt)
    for a, b2 in zip(dmod["layers"], fresh["layers"]):
        assert torch.equal(a["k_cache"], b2["k_cache"]) and torch.equal(a["v_cache"], b2["v_cache"])
    dm.close()


def test_decode_capacity_error(dev):
    m = wl.TINY_QWEN3
    weights = wl.model_weights(m)
    dm = gpu_model(q, m, upload_model(m, weights, dev))
    cap = m.layers[0].cap
    with pytest.raises(q.Q4Error) as e:
        dm.set_position(cap)
    assert e.value.status_name == "Q4_ERR_CAPACITY"
    dm.set_position(cap - 1)
    tok = torch.zeros(m.batch, dtype=torch.int32, device=dev)
    nxt = torch.empty_like(tok)
    dm.step(tok, nxt)
    with pytest.raises(q.Q4Error) as e:
        dm.step(tok, nxt)
    assert e.value.status_name == "Q4_ERR_CAPACITY"
    torch.cuda.synchronize()
    dm.close()
