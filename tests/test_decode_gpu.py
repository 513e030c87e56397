"""GPU decode step (HIP graph) against the fp64 oracle.

Per-op parity is checked in lockstep: the step is recomposed from the same
C-ABI calls, each call's output is compared with the oracle op fed the GPU's
own inputs, and the composition is checked to equal the library's step bit
for bit.  End to end, the greedy tokens must be identical to the oracle's at
every step; the logit NMSE and top-2 margins are reported.
"""
import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
from synth import workloads as wl

from decode_util import (gpu_model, lockstep_step, lockstep_step_variants, prefilled_caches, run_gpu,
                         run_oracle,
                         upload_model)

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


@pytest.mark.parametrize("shape", [wl.TINY_QWEN3, wl.TINY_GEMMA4], ids=lambda s: s.name)
def test_decode_lockstep_per_op(dev, shape):
    """Recompose one step from the C-ABI ops; check every op against the oracle
    fed the GPU's inputs, then check the composition equals decode_step_eager."""
    _say(f"lockstep {shape.name}")
    m = shape
    weights = wl.model_weights(m)
    dmod = upload_model(m, weights, dev)
    tok, nxt, logits, _ = lockstep_step(q, oracle, m, weights, dmod, dev, say=_say)

    # the library's own step runs the same kernels in the same order: bit-identical
    fresh = upload_model(m, weights, dev)
    dm = gpu_model(q, m, fresh)
    dm.set_position(m.start_pos)
    nxt2 = torch.empty_like(tok)
    lg2 = torch.empty((m.batch, m.vocab), dtype=torch.float32, device=dev)
    dm.step(tok, nxt2, lg2, eager=True)
    torch.cuda.synchronize()
    assert torch.equal(lg2, logits) and torch.equal(nxt2, nxt)
    for a, b2 in zip(dmod["layers"], fresh["layers"]):
        assert torch.equal(a["k_cache"], b2["k_cache"]) and torch.equal(a["v_cache"], b2["v_cache"])
    dm.close()


def test_decode_lockstep_per_op_variants(dev):
    """The Gemma-4 block variants at B = 1 (scaled gather, sandwich post-norms
    fused into the next projection, p-RoPE layers, GeGLU, soft cap): every op
    against the oracle fed the GPU's inputs, and the composition equal to
    decode_step_eager bit for bit."""
    m = wl.TINY_GEMMA4_EXACT_B1
    _say(f"lockstep {m.name}")
    weights = wl.model_weights(m)
    dmod = upload_model(m, weights, dev)
    tok, nxt, logits, rep = lockstep_step_variants(q, oracle, m, weights, dmod, dev, say=_say)
    assert any("post-norm" in k for k in rep) and any("p-RoPE" in k for k in rep)
    fresh = upload_model(m, weights, dev)
    dm = gpu_model(q, m, fresh)
    dm.set_position(m.start_pos)
    nxt2 = torch.empty_like(tok)
    lg2 = torch.empty((m.batch, m.vocab), dtype=torch.float32, device=dev)
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
