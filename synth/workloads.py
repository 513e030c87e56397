"""Shapes and seeded inputs of the workloads (no arithmetic of the method).

Workloads (sizes and value distributions as stated for each):
  * matvec_2048x6144   -- one Q4_0 matvec, K=2048 in, N=6144 out, B=1.
  * matvec_5376x21504  -- one Q4_0 matvec at the 31B FFN projection shape,
                          K=5376, N=21504 (65,028,096 weight bytes), B=1 and B=8.
  * attn_qwen3_1p7b    -- 28-layer GQA decode attention stack, 16 q / 8 kv heads,
                          head_dim 128, 4096 cached positions (N(0,1)), new token
                          at position 4096 with per-head RMSNorm (gains
                          U[0.8,1.2], eps 1e-6) and NeoX RoPE (theta 1e6).
  * decode_qwen3_4b    -- Qwen3-4B-shaped decode step: 36 layers, width 2560,
                          32 q / 8 kv heads, head_dim 128, SwiGLU FFN 9728,
                          Q8_0 tied table (vocab 151936), KV prefilled to 2048,
                          B=8, 16 greedy steps.
  * decode_gemma4_31b  -- Gemma-4-31B-shaped decode step: 60 layers, width 5376,
                          32 q heads, FFN 21504, pattern of 5 sliding-window
                          layers (16 kv heads, head_dim 256, window 1024) then 1
                          full layer (4 kv heads, head_dim 512, V from K),
                          Q8_0 vocab 262144, 8192 cached positions, B=1,
                          16 greedy steps.

Distributions: Q4_0 scales binary16 U[0.005, 0.02], codes uniform 0..15;
Q8_0 scales U[0.002, 0.01], codes U{-127..127}; activations and cache entries
fp32 N(0,1); norm gains fp32 U[0.8, 1.2]; start tokens uniform in [0, vocab).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

from . import normal_f32, q4_0_matrix, q8_0_matrix, tokens, uniform_f32

SEED_BASE = 20261202


@dataclass(frozen=True)
class MatvecWorkload:
    name: str
    n: int
    k: int
    batches: tuple
    seed: int


MATVEC_2048x6144 = MatvecWorkload("matvec_2048x6144", 6144, 2048, (1,), SEED_BASE + 0)
MATVEC_5376x21504 = MatvecWorkload("matvec_5376x21504", 21504, 5376, (1, 8), SEED_BASE + 1)


def matvec_inputs(w: MatvecWorkload, batch: int, copy: int = 0):
    """(W bytes [N, K/32*18], x [B, K] fp32).  ``copy`` selects an independently
    drawn weight copy (used to rotate weights out of the caches when timing)."""
    W = q4_0_matrix(w.seed, f"{w.name}.W{copy}", w.n, w.k)
    x = normal_f32(w.seed, f"{w.name}.x.B{batch}", (batch, w.k))
    return W, x


@dataclass(frozen=True)
class LayerShape:
    n_kv_heads: int
    head_dim: int
    window: int          # 0 = full attention
    rope_theta: float
    attn_scale: float
    v_from_k: bool
    cap: int             # cache slots per (sequence, kv head); slot = position % cap
    rope_dims: int = 0   # rotated dims (p-RoPE); 0 = the whole head


@dataclass(frozen=True)
class ModelShape:
    name: str
    d_model: int
    n_q_heads: int
    ffn: int
    vocab: int
    batch: int
    eps: float
    start_pos: int
    layers: tuple
    seed: int
    steps: int = 16
    # Gemma-4 block variants (defaults: the plain pre-norm SwiGLU block)
    ffn_act: str = "silu"       # or "gelu_tanh" (GeGLU)
    embed_scale: float = 0.0    # gathered embedding rows times this (0: unscaled)
    logit_softcap: float = 0.0  # logits c tanh(l / c) (0: none)
    sandwich: bool = False      # post-attention and post-FFN RMSNorm before the residual adds

    @property
    def n_layers(self):
        return len(self.layers)


def _qwen3(name, n_layers, d, hq, hkv, hd, ffn, vocab, batch, start, steps, seed):
    ly = LayerShape(hkv, hd, 0, 1e6, 1.0 / math.sqrt(hd), False, start + steps)
    return ModelShape(name, d, hq, ffn, vocab, batch, 1e-6, start, tuple([ly] * n_layers), seed,
                      steps)


def _gemma4(name, n_layers, d, hq, swa_hkv, swa_hd, window, full_hkv, full_hd, ffn, vocab,
            batch, start, steps, seed, exact=False):
    """exact: the Gemma-4 block variants the pages name -- p-RoPE (p = 0.25) on
    the full layers, GeGLU, sandwich norms, sqrt(d) embedding scale and a final
    logit soft cap (30, a reading: the pages give no value)."""
    layers = []
    for l in range(n_layers):
        if l % 6 == 5:
            layers.append(LayerShape(full_hkv, full_hd, 0, 1e6, 1.0, True, start + steps,
                                     full_hd // 4 if exact else 0))
        else:
            layers.append(LayerShape(swa_hkv, swa_hd, window, 1e4, 1.0, False, window))
    if not exact:
        return ModelShape(name, d, hq, ffn, vocab, batch, 1e-6, start, tuple(layers), seed, steps)
    return ModelShape(name, d, hq, ffn, vocab, batch, 1e-6, start, tuple(layers), seed, steps,
                      ffn_act="gelu_tanh", embed_scale=math.sqrt(d), logit_softcap=30.0,
                      sandwich=True)


QWEN3_4B = _qwen3("decode_qwen3_4b", 36, 2560, 32, 8, 128, 9728, 151936, 8, 2048, 16,
                  SEED_BASE + 3)
GEMMA4_31B = _gemma4("decode_gemma4_31b", 60, 5376, 32, 16, 256, 1024, 4, 512, 21504, 262144,
                     1, 8192, 16, SEED_BASE + 4)

# The 31B-shaped model decoding at a 128K-token context (full-attention
# caches of 131,088 slots); same weights as GEMMA4_31B.
GEMMA4_31B_128K = _gemma4("decode_gemma4_31b_128k", 60, 5376, 32, 16, 256, 1024, 4, 512, 21504,
                          262144, 1, 131072, 16, SEED_BASE + 4)

# Small models with the same structure, for parity tests the oracle finishes fast.
TINY_QWEN3 = _qwen3("tiny_qwen3", 2, 256, 4, 2, 64, 512, 1000, 3, 37, 4, 7001)
TINY_GEMMA4 = _gemma4("tiny_gemma4", 6, 256, 4, 2, 64, 16, 1, 128, 512, 1000, 2, 40, 4, 7002)
# The tiny Qwen3 structure with 20 sequences (three groups of 8 in the
# batched projections, the last one ragged).
TINY_QWEN3_B20 = _qwen3("tiny_qwen3_b20", 2, 256, 4, 2, 64, 512, 1000, 20, 37, 4, 7004)
# The tiny structure with the exact Gemma-4 block variants.
TINY_GEMMA4_EXACT = _gemma4("tiny_gemma4_exact", 6, 256, 4, 2, 64, 16, 1, 128, 512, 1000, 2, 40, 4,
                            7005, exact=True)
# The same with one sequence: the projections run on the vector kernels, which
# take the sandwich post-norms into the next projection's input.
TINY_GEMMA4_EXACT_B1 = _gemma4("tiny_gemma4_exact_b1", 6, 256, 4, 2, 64, 16, 1, 128, 512, 1000, 1, 40,
                               4, 7006, exact=True)
# The 31B shape with the exact Gemma-4 block variants (same matrices as
# GEMMA4_31B plus the post-norm gains).
GEMMA4_31B_EXACT = _gemma4("decode_gemma4_31b_exact", 60, 5376, 32, 16, 256, 1024, 4, 512, 21504,
                           262144, 1, 8192, 16, SEED_BASE + 4, exact=True)
# The tiny structure at a 128K-token context: its full-attention layer holds
# 2,049 chunks of 64 keys per sequence, so attention runs as multi-chunk splits.
TINY_GEMMA4_LONG = _gemma4("tiny_gemma4_long", 6, 256, 4, 2, 64, 16, 1, 128, 512, 1000, 2, 131072,
                           3, 7003)


def layer_rows(m: ModelShape, ly: LayerShape):
    nq = m.n_q_heads * ly.head_dim
    nk = ly.n_kv_heads * ly.head_dim
    return nq, nk, (0 if ly.v_from_k else nk)


def layer_weights(m: ModelShape, l: int):
    """Host arrays of layer ``l`` (its index in the full model) of the model."""
    s = m.seed
    ly = m.layers[l]
    nq, nk, nv = layer_rows(m, ly)
    w = dict(
        wqkv=q4_0_matrix(s, f"L{l}.wqkv", nq + nk + nv, m.d_model),
        wo=q4_0_matrix(s, f"L{l}.wo", m.d_model, nq),
        wgu=q4_0_matrix(s, f"L{l}.wgu", 2 * m.ffn, m.d_model),
        wd=q4_0_matrix(s, f"L{l}.wd", m.d_model, m.ffn),
        attn_norm=uniform_f32(s, f"L{l}.attn_norm", (m.d_model,), 0.8, 1.2),
        ffn_norm=uniform_f32(s, f"L{l}.ffn_norm", (m.d_model,), 0.8, 1.2),
        q_norm=uniform_f32(s, f"L{l}.q_norm", (ly.head_dim,), 0.8, 1.2),
        k_norm=uniform_f32(s, f"L{l}.k_norm", (ly.head_dim,), 0.8, 1.2),
    )
    if m.sandwich:
        w["post_attn_norm"] = uniform_f32(s, f"L{l}.post_attn_norm", (m.d_model,), 0.8, 1.2)
        w["post_ffn_norm"] = uniform_f32(s, f"L{l}.post_ffn_norm", (m.d_model,), 0.8, 1.2)
    return w


def model_weights(m: ModelShape, layer_ids=None):
    """Host arrays of every weight of the model (merged QKV and gate|up rows);
    with ``layer_ids`` only those layers (full-model indices), in that order."""
    s = m.seed
    ids = range(m.n_layers) if layer_ids is None else layer_ids
    return dict(
        embed=q8_0_matrix(s, "embed", m.vocab, m.d_model),
        final_norm=uniform_f32(s, "final_norm", (m.d_model,), 0.8, 1.2),
        layers=[layer_weights(m, l) for l in ids],
    )


def submodel(m: ModelShape, layer_ids, name=None):
    """The model restricted to the full-model layers ``layer_ids`` (same
    widths, vocabulary, batch and start position); pair it with
    ``model_weights(m, layer_ids)`` and the caches of those layers."""
    return replace(m, name=name or f"{m.name}_L" + "_".join(str(i) for i in layer_ids),
                   layers=tuple(m.layers[i] for i in layer_ids))


def prefilled_cache(m: ModelShape, l: int, which: str):
    """fp32 cache [B, Hkv, cap, hd] holding N(0,1) rows for positions < start_pos.

    Position p lives in slot p % cap; slots no prefilled position maps to are 0.
    """
    ly = m.layers[l]
    shape = (m.batch, ly.n_kv_heads, ly.cap, ly.head_dim)
    filled = min(m.start_pos, ly.cap)
    c = np.zeros(shape, dtype=np.float32)
    if filled:
        c[:, :, :filled, :] = normal_f32(m.seed, f"L{l}.{which}cache",
                                         (m.batch, ly.n_kv_heads, filled, ly.head_dim))
    return c


def start_tokens(m: ModelShape):
    return tokens(m.seed, "start_tokens", m.batch, m.vocab)


def oracle_spec(m: ModelShape, weights, caches):
    """The dict oracle.Model takes; ``caches`` is a list of (k, v) fp32 arrays."""
    layers = []
    for l, ly in enumerate(m.layers):
        w = weights["layers"][l]
        layers.append(dict(
            wqkv=w["wqkv"], wo=w["wo"], wgu=w["wgu"], wd=w["wd"],
            attn_norm=w["attn_norm"], ffn_norm=w["ffn_norm"], q_norm=w["q_norm"],
            k_norm=w["k_norm"], k_cache=caches[l][0], v_cache=caches[l][1],
            n_kv_heads=ly.n_kv_heads, head_dim=ly.head_dim, window=ly.window,
            rope_theta=ly.rope_theta, attn_scale=ly.attn_scale, v_from_k=ly.v_from_k,
            rope_dims=ly.rope_dims, post_attn_norm=w.get("post_attn_norm"),
            post_ffn_norm=w.get("post_ffn_norm")))
    return dict(d_model=m.d_model, n_q_heads=m.n_q_heads, ffn=m.ffn, vocab=m.vocab,
                batch=m.batch, eps=m.eps, embed=weights["embed"],
                final_norm=weights["final_norm"], layers=layers, ffn_act=m.ffn_act,
                embed_scale=m.embed_scale, logit_softcap=m.logit_softcap)


@dataclass(frozen=True)
class AttnStackWorkload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_cache: int
    rope_theta: float
    eps: float
    batches: tuple
    seed: int


ATTN_QWEN3_1P7B = AttnStackWorkload("attn_qwen3_1p7b", 28, 16, 8, 128, 4096, 1e6, 1e-6, (1, 8),
                                    SEED_BASE + 2)


def attn_layer_inputs(w: AttnStackWorkload, batch: int, l: int, cap: int = None):
    """Inputs of one layer: pre-norm q [B,Hq,hd], k/v [B,Hkv,hd], gains, and the
    fp32 caches [B,Hkv,cap,hd] with N(0,1) rows at positions < n_cache."""
    cap = cap or (w.n_cache + 1)
    s = w.seed
    tag = f"B{batch}.L{l}"
    q = normal_f32(s, f"{tag}.q", (batch, w.n_q_heads, w.head_dim))
    k = normal_f32(s, f"{tag}.k", (batch, w.n_kv_heads, w.head_dim))
    v = normal_f32(s, f"{tag}.v", (batch, w.n_kv_heads, w.head_dim))
    qn = uniform_f32(s, f"L{l}.q_norm", (w.head_dim,), 0.8, 1.2)
    kn = uniform_f32(s, f"L{l}.k_norm", (w.head_dim,), 0.8, 1.2)
    kc = np.zeros((batch, w.n_kv_heads, cap, w.head_dim), dtype=np.float32)
    vc = np.zeros_like(kc)
    kc[:, :, :w.n_cache] = normal_f32(s, f"{tag}.kcache", (batch, w.n_kv_heads, w.n_cache,
                                                             w.head_dim))
    vc[:, :, :w.n_cache] = normal_f32(s, f"{tag}.vcache", (batch, w.n_kv_heads, w.n_cache,
                                                             w.head_dim))
    return q, k, v, qn, kn, kc, vc
