"""Full-size workloads on the GPU against the fp64 oracle.

* Decode: the 4B-shaped model at B = 8 and the 31B-shaped model at B = 1, 16
  greedy steps through the captured graph, from the prefilled position.  The
  oracle's tokens, margins, sampled logits and, at the first and the last
  step, every logit of the vocabulary were written by
  tests/golden/make_decode_oracle.py (oracle only).  The GPU tokens must be
  identical at every step; at the sampled indices (the oracle's 8 largest plus
  24 fixed ones) of every step and at every index of the first and last steps
  the GPU logits must agree to a small fraction of the logits' RMS, and the
  whole-vocabulary NMSE must stay below 1e-8.
* Lockstep at full size: one step of a two-layer model made of layer 0 (a
  sliding-window layer, its 1,024-slot ring wrapping at position 8192) and
  layer 5 (a full-attention layer) of the 31B shape at B = 1 (vector kernels,
  K split 1, 2 and 4 ways), and of layer 0 of the 4B shape at B = 8 (matrix
  cores), recomposed from the C-ABI calls with every op checked against the
  oracle fed the GPU's own inputs, then checked to equal the library's own
  step bit for bit.
* Attention: the 28-layer Qwen3-1.7B-shaped stack at n_cache = 4096 (QK-norm,
  RoPE at position 4096, KV append, attention over 4097 keys), every head of
  every layer at B = 1 and of three layers at B = 8, each checked against the
  oracle fed the GPU's own normalised q and appended cache row.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
from q4_quantized_matvec_amd._lib import kv_layout_of
from synth import workloads as wl

from decode_util import (gpu_model, lockstep_step, lockstep_step_variants, prefilled_caches, run_gpu,
                         upload_model)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("shape", [wl.QWEN3_4B, wl.GEMMA4_31B], ids=lambda s: s.name)
def test_decode_fullsize_matches_oracle(dev, shape):
    with open(os.path.join(GOLDEN, f"{shape.name}_oracle.json")) as f:
        gold = json.load(f)
    assert gold["seed"] == shape.seed and gold["steps"] == shape.steps
    assert gold["start_tokens"] == wl.start_tokens(shape).tolist()
    _say(f"decode {shape.name}: generating weights")
    weights = wl.model_weights(shape)
    dmod = upload_model(shape, weights, dev)
    del weights
    _say(f"decode {shape.name}: {shape.steps} steps")
    toks, logits = run_gpu(q, shape, dmod, shape.steps)
    del dmod
    torch.cuda.empty_cache()
    worst = 0.0
    for s in range(shape.steps):
        assert toks[s].tolist() == gold["tokens"][s], f"step {s}: tokens differ"
        for b in range(shape.batch):
            idx = np.array(gold["sample_idx"][s][b])
            ref = np.array(gold["sample_logits"][s][b])
            rms = np.sqrt(gold["logits_sq_sum"][s][b] / shape.vocab)
            err = np.abs(logits[s, b, idx].astype(np.float64) - ref).max() / rms
            worst = max(worst, err)
    _say(f"  tokens identical over {shape.steps} steps; sampled max |dlogit| / rms = {worst:.3e}; "
         f"min oracle margin {np.min(gold['margins']):.4f}")
    assert worst < 1e-4
    # every logit of the vocabulary at the first and the last step
    assert gold["full_logit_steps"] == [0, shape.steps - 1]
    for s in gold["full_logit_steps"]:
        ref = np.load(os.path.join(GOLDEN, f"{shape.name}_logits_s{s:02d}.npy")).astype(np.float64)
        assert ref.shape == (shape.batch, shape.vocab)
        got = logits[s].astype(np.float64)
        for b in range(shape.batch):
            d = got[b] - ref[b]
            rms = np.sqrt(np.mean(ref[b] ** 2))
            nmse = float((d ** 2).sum() / (ref[b] ** 2).sum())
            corr = float(np.corrcoef(got[b], ref[b])[0, 1])
            mx = float(np.abs(d).max() / rms)
            mae = float(np.abs(d).mean() / rms)
            _say(f"  step {s} seq {b}: all {shape.vocab} logits: corr {corr:.12f} nmse {nmse:.3e} "
                 f"mean |d|/rms {mae:.3e} max |d|/rms {mx:.3e}")
            assert nmse <= 1e-8, f"step {s} seq {b}: nmse {nmse:.3e}"
            assert mx <= 1e-4, f"step {s} seq {b}: max |dlogit| / rms {mx:.3e}"


# (workload, full-model layer indices): 31B layers 0 (sliding window, ring) and
# 5 (full attention, V from K); 4B layer 0 at B = 8
_LOCKSTEP = [(wl.GEMMA4_31B, (0, 5)), (wl.QWEN3_4B, (0,))]


@pytest.mark.parametrize("shape,ids", _LOCKSTEP, ids=lambda v: v.name if hasattr(v, "name") else
                         "L" + "_".join(map(str, v)))
def test_lockstep_fullsize(dev, shape, ids):
    m = wl.submodel(shape, ids)
    _say(f"lockstep {m.name}: B={m.batch} at position {m.start_pos}, generating weights")
    weights = wl.model_weights(shape, ids)
    caches = prefilled_caches(shape, layer_ids=ids)
    dmod = upload_model(m, weights, dev, caches=caches)
    tok, nxt, logits, rep = lockstep_step(q, oracle, m, weights, dmod, dev, say=_say)
    _say("  worst err/tol per op: " + ", ".join(f"{k} {v:.2e}" for k, v in rep.items()))
    # the library's own step (eager) on a fresh copy: same kernels, same order
    fresh = upload_model(m, weights, dev, caches=caches)
    dm = gpu_model(q, m, fresh)
    dm.set_position(m.start_pos)
    nxt2 = torch.empty_like(tok)
    lg2 = torch.empty((m.batch, m.vocab), dtype=torch.float32, device=dev)
    dm.step(tok, nxt2, lg2, eager=True)
    torch.cuda.synchronize()
    assert torch.equal(lg2, logits) and torch.equal(nxt2, nxt)
    for a, b2 in zip(dmod["layers"], fresh["layers"]):
        assert torch.equal(a["k_cache"], b2["k_cache"]) and torch.equal(a["v_cache"], b2["v_cache"])
    # and the captured graph of that step gives the same bits
    dm.set_position(m.start_pos)
    for a, b2 in zip(dmod["layers"], fresh["layers"]):
        b2["k_cache"].copy_(a["k_cache"])
        b2["v_cache"].copy_(a["v_cache"])
    lg3 = torch.empty_like(lg2)
    dm.step(tok, nxt2, lg3)
    torch.cuda.synchronize()
    assert torch.equal(lg3, logits)
    dm.close()
    del dmod, fresh
    torch.cuda.empty_cache()


def test_lockstep_fullsize_variants(dev):
    """The 31B shape with the Gemma-4 block variants, layers 0 (sliding window,
    1,024-slot ring at position 8,192) and 5 (full attention, p-RoPE over 128
    of 512 dims, V from K): the scaled gather, the sandwich post-norms fused
    into the next projection (K = 5,376 vector kernel, GeGLU output over
    2 x 21,504 rows), the K-split down projection without a residual, the
    last post-norm, the soft-capped 262,144 logits; each op against the
    oracle fed the GPU's inputs, then the library's own eager step and its
    graph on a fresh copy give the same bits."""
    shape, ids = wl.GEMMA4_31B_EXACT, (0, 5)
    m = wl.submodel(shape, ids)
    _say(f"lockstep {m.name}: B={m.batch} at position {m.start_pos}, generating weights")
    weights = wl.model_weights(shape, ids)
    caches = prefilled_caches(shape, layer_ids=ids)
    dmod = upload_model(m, weights, dev, caches=caches)
    tok, nxt, logits, rep = lockstep_step_variants(q, oracle, m, weights, dmod, dev, say=_say)
    _say("  worst err/tol per op: " + ", ".join(f"{k} {v:.2e}" for k, v in rep.items()))
    fresh = upload_model(m, weights, dev, caches=caches)
    dm = gpu_model(q, m, fresh)
    dm.set_position(m.start_pos)
    nxt2 = torch.empty_like(tok)
    lg2 = torch.empty((m.batch, m.vocab), dtype=torch.float32, device=dev)
    dm.step(tok, nxt2, lg2, eager=True)
    torch.cuda.synchronize()
    assert torch.equal(lg2, logits) and torch.equal(nxt2, nxt)
    dm.set_position(m.start_pos)
    for a, b2 in zip(dmod["layers"], fresh["layers"]):
        b2["k_cache"].copy_(a["k_cache"])
        b2["v_cache"].copy_(a["v_cache"])
    lg3 = torch.empty_like(lg2)
    dm.step(tok, nxt2, lg3)
    torch.cuda.synchronize()
    assert torch.equal(lg3, logits)
    dm.close()
    del dmod, fresh
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch,layers", [(1, tuple(range(28))), (8, (0, 13, 27))],
                         ids=["B1_all_layers", "B8_three_layers"])
def test_attention_stack_qwen3_1p7b(dev, batch, layers):
    w = wl.ATTN_QWEN3_1P7B
    hq, hkv, hd, pos = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_cache
    n = pos + 1
    pos_d = torch.tensor([pos, n], dtype=torch.int64, device=dev)
    worst = 0.0
    for l in layers:
        _say(f"attention stack B={batch} layer {l}")
        qh, kh, vh, qn, kn, kc, vc = wl.attn_layer_inputs(w, batch, l)
        qd = torch.from_numpy(qh.reshape(batch, hq * hd).copy()).to(dev)
        kd = torch.from_numpy(kh.reshape(batch, hkv * hd).copy()).to(dev)
        vd = torch.from_numpy(vh.reshape(batch, hkv * hd).copy()).to(dev)
        kcd = torch.from_numpy(kc).to(dev)
        vcd = torch.from_numpy(vc).to(dev)
        kv = kv_layout_of(kcd)
        q.qk_norm_rope(qd, hq * hd, kd, vd, hkv * hd, torch.from_numpy(qn).to(dev),
                       torch.from_numpy(kn).to(dev), hq, kv, pos_d[0:1], w.rope_theta, w.eps,
                       False, kcd, vcd)
        ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, 0), dtype=torch.uint8, device=dev)
        out = torch.empty((batch, hq * hd), dtype=torch.float32, device=dev)
        q.gqa_decode_attn(qd, hq * hd, hq, kcd, vcd, kv, pos_d[1:2], 0, 1.0 / np.sqrt(hd), out,
                          hq * hd, ws)
        torch.cuda.synchronize()
        qg = qd.cpu().numpy().astype(np.float64).reshape(batch, hq, hd)
        newk = kcd[:, :, pos].cpu().numpy().astype(np.float64)
        newv = vcd[:, :, pos].cpu().numpy().astype(np.float64)
        og = out.cpu().numpy().astype(np.float64).reshape(batch, hq, hd)
        for b in range(batch):
            # the appended rows and the rotated query against the oracle
            q_ref = oracle.rope_neox(oracle.rmsnorm(qh[b], qn, w.eps), pos, w.rope_theta)
            k_ref = oracle.rope_neox(oracle.rmsnorm(kh[b], kn, w.eps), pos, w.rope_theta)
            assert np.all(np.abs(qg[b] - q_ref) <= 2e-4 * np.abs(q_ref) + 2e-5)
            assert np.all(np.abs(newk[b] - k_ref) <= 2e-4 * np.abs(k_ref) + 2e-5)
            assert np.array_equal(newv[b], vh[b].astype(np.float64))
            keys = np.concatenate([kc[b, :, :pos].transpose(1, 0, 2), newk[b][None]], axis=0)
            vals = np.concatenate([vc[b, :, :pos].transpose(1, 0, 2), newv[b][None]], axis=0)
            o, bound = oracle.gqa_attention(qg[b], keys, vals, 0, 1.0 / np.sqrt(hd))
            ratio = float((np.abs(og[b] - o) / (2e-4 * bound + 1e-6)).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"layer {l} seq {b}: max err/tol {ratio:.3e}"
        del kcd, vcd
    _say(f"  worst err/tol {worst:.3e}")
