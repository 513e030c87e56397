"""Helpers shared by the decode-step GPU tests and the benchmark: upload a
synthetic model to the device and run GPU / oracle decode loops."""
import numpy as np

from synth import workloads as wl


def upload_model(m, weights, dev, caches=None):
    """Device tensors of every weight and a prefilled cache per layer
    (``caches``: per layer a (k, v) pair of host arrays or device tensors)."""
    import torch
    layers = []
    for l, ly in enumerate(m.layers):
        w = weights["layers"][l]
        if caches is None:
            kc = wl.prefilled_cache(m, l, "k")
            vc = wl.prefilled_cache(m, l, "v")
        else:
            kc, vc = caches[l]
        as_dev = lambda a: a if isinstance(a, torch.Tensor) else torch.from_numpy(a).to(dev)
        layers.append(dict(
            wqkv=torch.from_numpy(w["wqkv"]).to(dev), wo=torch.from_numpy(w["wo"]).to(dev),
            wgu=torch.from_numpy(w["wgu"]).to(dev), wd=torch.from_numpy(w["wd"]).to(dev),
            attn_norm=torch.from_numpy(w["attn_norm"]).to(dev),
            ffn_norm=torch.from_numpy(w["ffn_norm"]).to(dev),
            q_norm=torch.from_numpy(w["q_norm"]).to(dev), k_norm=torch.from_numpy(w["k_norm"]).to(dev),
            k_cache=as_dev(kc), v_cache=as_dev(vc),
            n_kv_heads=ly.n_kv_heads, head_dim=ly.head_dim, window=ly.window,
            rope_theta=ly.rope_theta, attn_scale=ly.attn_scale, v_from_k=ly.v_from_k,
            rope_dims=ly.rope_dims))
        for key in ("post_attn_norm", "post_ffn_norm"):
            if key in w:
                layers[-1][key] = torch.from_numpy(w[key]).to(dev)
    return dict(embed=torch.from_numpy(weights["embed"]).to(dev),
                final_norm=torch.from_numpy(weights["final_norm"]).to(dev), layers=layers)


def gpu_model(q, m, dev_model):
    return q.DecodeModel(d_model=m.d_model, n_q_heads=m.n_q_heads, ffn=m.ffn, vocab=m.vocab,
                         batch=m.batch, eps=m.eps, embed=dev_model["embed"],
                         final_norm=dev_model["final_norm"], layers=dev_model["layers"],
                         ffn_act=m.ffn_act, embed_scale=m.embed_scale,
                         logit_softcap=m.logit_softcap)


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


def prefilled_caches(m, kv16=False):
    """Host caches of every layer from the workload recipe; kv16 rounds them
    to the nearest binary16 (numpy's conversion)."""
    out = []
    for l in range(m.n_layers):
        k, v = wl.prefilled_cache(m, l, "k"), wl.prefilled_cache(m, l, "v")
        if kv16:
            k, v = k.astype(np.float16), v.astype(np.float16)
        out.append((k, v))
    return out


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
