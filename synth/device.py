"""Device copies of the synthetic workloads (torch tensors on a GPU).

Only uploads: the seeded host arrays of ``synth.workloads`` are copied to the
device as they are, and the prefilled KV caches are laid out as the workload
recipe says.  Nothing here computes any part of the method, and nothing here
imports the library or the oracle.
"""
from __future__ import annotations

import numpy as np

from . import workloads as wl


def prefilled_caches(m, kv16=False, layer_ids=None):
    """Host caches of every layer (or of the full-model layer indices
    ``layer_ids``) from the workload recipe; ``kv16`` rounds them to the
    nearest binary16 (numpy's conversion)."""
    ids = range(m.n_layers) if layer_ids is None else layer_ids
    out = []
    for l in ids:
        k, v = wl.prefilled_cache(m, l, "k"), wl.prefilled_cache(m, l, "v")
        if kv16:
            k, v = k.astype(np.float16), v.astype(np.float16)
        out.append((k, v))
    return out


def upload_model(m, weights, dev, caches=None):
    """Device tensors of every weight and a prefilled cache per layer
    (``caches``: per layer a (k, v) pair of host arrays or device tensors;
    default: the recipe's caches of the model's own layers)."""
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


def model_kwargs(m, dev_model):
    """Keyword arguments of the binding's DecodeModel for an uploaded model."""
    return dict(d_model=m.d_model, n_q_heads=m.n_q_heads, ffn=m.ffn, vocab=m.vocab,
                batch=m.batch, eps=m.eps, embed=dev_model["embed"],
                final_norm=dev_model["final_norm"], layers=dev_model["layers"],
                ffn_act=m.ffn_act, embed_scale=m.embed_scale, logit_softcap=m.logit_softcap)
