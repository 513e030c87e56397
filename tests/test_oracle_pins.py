"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible slip in the oracle (dropped term, wrong
sign, swapped nibbles, transposed operand, wrong head mapping, wrong RoPE
pairing, wrong window edge) fails at least one of them.  Nothing here compares
the oracle with a copy of its own formula or with the HIP path.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_block():
    with open(os.path.join(GOLDEN, "q4_0_hand_block.json")) as f:
        g = json.load(f)
    blk = bytes.fromhex(g["block_hex"]) + bytes.fromhex(g["payload_hex"])
    assert len(blk) == 18
    return np.frombuffer(blk, dtype=np.uint8).copy(), g


# ----------------------------------------------------------------- binary16
def test_half_every_bit_pattern():
    """All 65,536 binary16 patterns against numpy's IEEE conversion."""
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # and the sign of zero
    assert math.copysign(1.0, oracle.half_to_double(0x8000)) == -1.0


# ----------------------------------------------------------------- Q4_0
def test_q4_0_hand_block_weights():
    blk, g = _hand_block()
    w = oracle.q4_0_dequant(blk, 1, 32)[0]
    assert w.tolist() == g["weights"]


def test_q4_0_hand_block_matvec_cases():
    blk, g = _hand_block()
    k = np.arange(32, dtype=np.float64)
    xs = {"ones": np.ones(32), "k_squared": k * k}
    for case in g["cases"]:
        y, _ = oracle.q4_0_matvec(blk, 1, 32, xs[case["x"]])
        assert y[0, 0] == case["y"], case
    # unit vectors recover each weight exactly; e_0 and e_16 tell the nibbles apart
    eye = np.eye(32)
    y, _ = oracle.q4_0_matvec(blk, 1, 32, eye)
    assert y[:, 0].tolist() == g["weights"]
    assert y[0, 0] == -0.5 and y[16, 0] == 0.4375


def test_q4_0_code_eight_is_zero_and_scale_little_endian():
    blk = np.zeros(18, dtype=np.uint8)
    blk[0:2] = [0x00, 0x3C]          # 0x3C00 = 1.0 little-endian
    blk[2:] = 0x88                   # every code 8 -> weight 0
    assert np.all(oracle.q4_0_dequant(blk, 1, 32) == 0.0)
    blk[2:] = 0xFF                   # every code 15 -> weight 7 * d
    assert np.all(oracle.q4_0_dequant(blk, 1, 32) == 7.0)
    blk[2:] = 0x00                   # every code 0 -> weight -8 * d
    assert np.all(oracle.q4_0_dequant(blk, 1, 32) == -8.0)


def _expand_codes_q4(w_bytes, n_rows, k):
    """Integer codes of a Q4_0 matrix, element order per the format statement."""
    blocks = w_bytes.reshape(n_rows, k // 32, 18)
    qs = blocks[:, :, 2:]
    codes = np.concatenate([qs & 0x0F, qs >> 4], axis=2)      # elements 0..15, 16..31
    return codes.reshape(n_rows, k).astype(np.int64)


def test_q4_0_matvec_integer_exact():
    """Power-of-two scale and integer x: the result is exact in int64 arithmetic."""
    rng = np.random.default_rng(7)
    n_rows, k = 13, 96
    w = synth.q4_0_matrix(11, "int-exact", n_rows, k)
    blocks = w.reshape(n_rows, k // 32, 18)
    blocks[:, :, 0] = 0x00
    blocks[:, :, 1] = 0x30            # 0x3000 = 0.125
    x = rng.integers(-50, 51, size=(3, k))
    codes = _expand_codes_q4(w, n_rows, k)
    exact = (x @ (codes - 8).T)       # int64, exact
    y, terms = oracle.q4_0_matvec(w, n_rows, k, x.astype(np.float64))
    assert np.array_equal(y, exact * 0.125)
    assert np.array_equal(terms, np.abs(x)[:, None, :].__mul__(np.abs(codes - 8)[None]).sum(-1) * 0.125)


def test_q4_0_vs_q8_0_cross_encoding():
    """A Q4_0 matrix re-encoded as Q8_0 (same scale, code - 8 per element) gives
    bit-identical products: catches a nibble-order or offset slip in either path."""
    n_rows, k = 9, 256
    w4 = synth.q4_0_matrix(3, "cross", n_rows, k)
    codes = _expand_codes_q4(w4, n_rows, k) - 8
    b4 = w4.reshape(n_rows, k // 32, 18)
    w8 = np.empty((n_rows, k // 32, 34), dtype=np.uint8)
    w8[:, :, 0:2] = b4[:, :, 0:2]
    w8[:, :, 2:] = codes.reshape(n_rows, k // 32, 32).astype(np.int8).view(np.uint8)
    x = synth.normal_f32(3, "cross-x", (4, k))
    y4, t4 = oracle.q4_0_matvec(w4, n_rows, k, x)
    y8, t8 = oracle.q8_0_matvec(w8.reshape(n_rows, -1), n_rows, k, x)
    assert np.array_equal(y4, y8) and np.array_equal(t4, t8)


@pytest.mark.parametrize("n_rows,k,batch", [(67, 32, 1), (67, 64, 3), (33, 256, 8), (5, 288, 2)])
def test_q4_0_matvec_matches_dense_product(n_rows, k, batch):
    """Brute force on tiny shapes (with non-multiple row tails): the blocked
    matvec equals a dense fp64 product of the dequantised matrix."""
    w = synth.q4_0_matrix(5, f"dense-{n_rows}-{k}", n_rows, k)
    x = synth.normal_f32(5, f"dense-x-{n_rows}-{k}", (batch, k)).astype(np.float64)
    r = synth.normal_f32(5, f"dense-r-{n_rows}-{k}", (batch, n_rows)).astype(np.float64)
    dense = oracle.q4_0_dequant(w, n_rows, k)
    y, terms = oracle.q4_0_matvec(w, n_rows, k, x, res=r)
    ref = x @ dense.T + r
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(terms, np.abs(x) @ np.abs(dense).T + np.abs(r), rtol=1e-13)
    # transposed-operand slip: the dense product with W (not W^T) has another shape
    assert dense.shape == (n_rows, k)


def test_q4_0_byte_count_fact():
    """Research record, buffer-ownership section: 5376 x 21504 Q4_0 = 65,028,096 bytes."""
    w = synth.q4_0_matrix(1, "fact", 4, 5376)
    assert w.shape[1] * 21504 == 65_028_096


# ----------------------------------------------------------------- Q8_0
def test_q8_0_hand_block():
    blk = np.zeros(34, dtype=np.uint8)
    blk[0:2] = [0x00, 0x38]                      # 0x3800 = 0.5
    codes = np.array([(-1) ** j * j for j in range(32)], dtype=np.int8)
    codes[31] = -127
    blk[2:] = codes.view(np.uint8)
    w = oracle.q8_0_dequant(blk, 1, 32)[0]
    assert w.tolist() == [0.5 * float(c) for c in codes]
    assert w[31] == -63.5 and w[2] == 1.0 and w[3] == -1.5


def test_q8_0_gather_is_row_of_table():
    v, k = 50, 64
    t = synth.q8_0_matrix(2, "gather", v, k)
    tok = np.array([0, 49, 7, 7], dtype=np.int32)
    x = oracle.q8_0_gather(t, v, k, tok)
    dense = oracle.q8_0_dequant(t, v, k)
    assert np.array_equal(x, dense[tok])
    # and equals the product with a unit vector on the output side
    y, _ = oracle.q8_0_matvec(t, v, k, np.eye(k))
    assert np.array_equal(y.T[tok], x)


# ----------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_gain_invariant():
    x = synth.normal_f32(4, "rms", (5, 300)).astype(np.float64) * 3.0
    eps = 1e-6
    y = oracle.rmsnorm(x, None, eps)
    ms = (x * x).mean(axis=1)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)


def test_rmsnorm_constant_row_and_hand_case():
    w = np.array([0.5, 1.0, 2.0, -1.0])
    c, eps = 3.0, 1e-6
    y = oracle.rmsnorm(np.full(4, c), w, eps)
    assert np.allclose(y, w * c / math.sqrt(c * c + eps), rtol=1e-15)
    y = oracle.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt(12.5)
    assert np.allclose(y, [3.0 / r, 8.0 / r], rtol=1e-15)


def test_rmsnorm_scale_invariance_without_eps():
    x = synth.normal_f32(4, "rms2", (300,)).astype(np.float64)
    w = synth.uniform_f32(4, "rms2w", (300,), 0.8, 1.2)
    a = oracle.rmsnorm(x, w, 0.0)
    assert np.allclose(oracle.rmsnorm(x * 1e3, w, 0.0), a, rtol=1e-13)
    assert np.allclose(oracle.rmsnorm(-x * 0.25, w, 0.0), -a, rtol=1e-13)


# ----------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = synth.normal_f32(6, "rope0", (3, 128)).astype(np.float64)
    assert np.array_equal(oracle.rope_neox(x, 0, 1e6), x)


def test_rope_one_pair_closed_form():
    """hd = 2: the single pair rotates by exactly pos radians."""
    for pos in (1, 7, 4096, 8200):
        y = oracle.rope_neox(np.array([1.0, 0.0]), pos, 1e6)
        assert y[0] == math.cos(pos) and y[1] == math.sin(pos)


def test_rope_neox_pairing_and_frequency():
    """hd = 4: element 1 pairs with element 3 (NeoX half split, not adjacent
    pairs) and turns at theta^(-2/4) per position."""
    theta, pos = 10000.0, 3
    y = oracle.rope_neox(np.array([0.0, 1.0, 0.0, 0.0]), pos, theta)
    a = pos * theta ** (-0.5)
    assert abs(y[1] - math.cos(a)) < 1e-15 and abs(y[3] - math.sin(a)) < 1e-15
    assert y[0] == 0.0 and y[2] == 0.0


def test_rope_norm_and_relative_position():
    hd = 128
    q = synth.normal_f32(6, "rq", (hd,)).astype(np.float64)
    k = synth.normal_f32(6, "rk", (hd,)).astype(np.float64)
    rq = oracle.rope_neox(q, 4096, 1e6)
    h = hd // 2
    assert np.allclose(rq[:h] ** 2 + rq[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-13)
    d1 = oracle.rope_neox(q, 900, 1e6) @ oracle.rope_neox(k, 700, 1e6)
    d2 = oracle.rope_neox(q, 250, 1e6) @ oracle.rope_neox(k, 50, 1e6)
    assert abs(d1 - d2) < 1e-11 * (np.abs(q) @ np.abs(k))


# ----------------------------------------------------------------- SwiGLU
def test_swiglu_values():
    g = np.array([0.0, 1.0, 40.0, -40.0, -1.0])
    u = np.array([5.0, 1.0, 1.0, 1.0, 2.0])
    h = oracle.swiglu(g, u)
    assert h[0] == 0.0
    assert abs(h[1] - 0.7310585786300049) < 1e-16
    assert abs(h[2] - 40.0) < 1e-15
    assert abs(h[3]) < 1e-15 and h[3] < 0
    assert abs(h[4] - 2.0 * (-1.0 / (1.0 + math.e))) < 1e-15


# ----------------------------------------------------------------- argmax
def test_argmax_ties_and_margin():
    i, m = oracle.argmax(np.array([1.0, 3.0, 3.0, 2.0]))
    assert i == 1 and m == 0.0
    i, m = oracle.argmax(np.array([-5.0, -1.0, -2.0]))
    assert i == 1 and m == 1.0
    v = synth.normal_f32(8, "am", (10000,)).astype(np.float64)
    i, m = oracle.argmax(v)
    assert i == max(range(v.size), key=lambda j: (v[j], -j))
    s = sorted(v.tolist())
    assert m == s[-1] - s[-2]


# ----------------------------------------------------------------- attention
def _attn_inputs(seed, hq, hkv, hd, n):
    q = synth.normal_f32(seed, "aq", (hq, hd)).astype(np.float64)
    k = synth.normal_f32(seed, "ak", (n, hkv, hd)).astype(np.float64)
    v = synth.normal_f32(seed, "av", (n, hkv, hd)).astype(np.float64)
    return q, k, v


def _attn_brute(q, k, v, window, scale):
    """Pure-Python loops over a tiny case, straight from the softmax definition."""
    hq, hd = q.shape
    n, hkv, _ = k.shape
    group = hq // hkv
    lo = max(0, n - window) if window else 0
    out = np.zeros((hq, hd))
    for h in range(hq):
        g = h // group
        s = [scale * sum(q[h, i] * k[j, g, i] for i in range(hd)) for j in range(lo, n)]
        mx = max(s)
        e = [math.exp(t - mx) for t in s]
        z = sum(e)
        for d in range(hd):
            out[h, d] = sum(e[j - lo] / z * v[j, g, d] for j in range(lo, n))
    return out


@pytest.mark.parametrize("window", [0, 1, 3, 8])
def test_attention_brute_force_small(window):
    q, k, v = _attn_inputs(1, 4, 2, 8, 6)
    o, _ = oracle.gqa_attention(q, k, v, window, 0.3)
    assert np.allclose(o, _attn_brute(q, k, v, window, 0.3), rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    q, k, v = _attn_inputs(2, 8, 2, 16, 9)
    # one key: the output is that key's value row
    o, _ = oracle.gqa_attention(q, k[:1], v[:1], 0, 1.0)
    assert np.allclose(o, np.repeat(v[0], 4, axis=0), rtol=1e-15)
    # window 1: only the newest position is seen
    o, _ = oracle.gqa_attention(q, k, v, 1, 1.0)
    assert np.allclose(o, np.repeat(v[-1], 4, axis=0), rtol=1e-15)
    # equal keys: uniform weights, output = mean of the values in the window
    ke = np.repeat(k[:1], 9, axis=0)
    o, _ = oracle.gqa_attention(q, ke, v, 0, 1.0)
    assert np.allclose(o, np.repeat(v.mean(axis=0), 4, axis=0), rtol=1e-13)
    o, _ = oracle.gqa_attention(q, ke, v, 4, 1.0)
    assert np.allclose(o, np.repeat(v[-4:].mean(axis=0), 4, axis=0), rtol=1e-13)
    # constant values: weights sum to one
    vc = np.full_like(v, 2.5)
    o, _ = oracle.gqa_attention(q, k, vc, 0, 0.7)
    assert np.allclose(o, 2.5, rtol=1e-15)
    # window >= n equals the full cache
    a, _ = oracle.gqa_attention(q, k, v, 9, 0.7)
    b, _ = oracle.gqa_attention(q, k, v, 0, 0.7)
    assert np.array_equal(a, b)


def test_attention_head_group_mapping():
    """Query head h reads kv head h // (Hq / Hkv)."""
    hq, hkv, hd, n = 8, 4, 4, 5
    q, k, _ = _attn_inputs(3, hq, hkv, hd, n)
    v = np.zeros((n, hkv, hd))
    for g in range(hkv):
        v[:, g, :] = g
    o, _ = oracle.gqa_attention(q, k, v, 0, 1.0)
    assert np.allclose(o[:, 0], [h // 2 for h in range(hq)], rtol=1e-15)


def test_attention_mha_equals_per_head():
    q, k, v = _attn_inputs(4, 3, 3, 8, 7)
    o, _ = oracle.gqa_attention(q, k, v, 0, 0.5)
    for h in range(3):
        oh, _ = oracle.gqa_attention(q[h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 0, 0.5)
        assert np.array_equal(oh[0], o[h])


def test_attention_two_key_closed_form():
    q = np.array([[1.0, 2.0]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = np.array([[[10.0, 0.0]], [[0.0, 4.0]]])
    o, _ = oracle.gqa_attention(q, k, v, 0, 0.5)
    e1, e2 = math.exp(0.5), math.exp(1.0)
    assert np.allclose(o[0], [10.0 * e1 / (e1 + e2), 4.0 * e2 / (e1 + e2)], rtol=1e-15)


def test_attention_chunk_merge_composition():
    """Attention over all keys equals the merge of attention over disjoint chunks,
    each weighted by its share of the softmax mass (the split-K identity)."""
    q, k, v = _attn_inputs(5, 2, 1, 16, 40)
    scale = 0.25
    full, _ = oracle.gqa_attention(q, k, v, 0, scale)
    cuts = [0, 7, 8, 25, 40]
    for h in range(2):
        num = np.zeros(16)
        den = 0.0
        for a, b in zip(cuts[:-1], cuts[1:]):
            oc, _ = oracle.gqa_attention(q[h:h + 1], k[a:b], v[a:b], 0, scale)
            s = scale * (k[a:b, 0] @ q[h])
            mass = np.exp(s).sum()
            num += mass * oc[0]
            den += mass
        assert np.allclose(num / den, full[h], rtol=1e-12)


# ---------------------------------------------------------------- binary16 caches
def test_double_to_half_matches_numpy_rounding():
    """The oracle's nearest-binary16 rounding against numpy's float64 ->
    float16 conversion (an independent implementation of the same IEEE
    rounding): random magnitudes across every binade, subnormals, exact ties,
    the overflow threshold, signed zero and NaN."""
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(20000) * np.exp2(rng.integers(-30, 17, 20000)))
    # midpoints between neighbouring halves (ties go to the even fraction)
    for h in rng.integers(0, 0x7BFF, 2000):
        a = np.array([h, h + 1], dtype=np.uint16).view(np.float16).astype(np.float64)
        vals.append((a[0] + a[1]) / 2)
        vals.append(-(a[0] + a[1]) / 2)
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
             2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25]
    got = np.array([oracle.double_to_half(v) for v in vals], dtype=np.uint16)
    exp = np.array(vals, dtype=np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp)
    nan = oracle.double_to_half(float("nan"))
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_double_to_half_inverts_half_to_double():
    for h in range(0x10000):
        if (h & 0x7C00) == 0x7C00 and (h & 0x3FF):
            continue  # NaN payloads are not preserved
        assert oracle.double_to_half(oracle.half_to_double(h)) == h


def test_decode_f16_cache_appends_rounded_rows():
    """One step with binary16 caches: layer 0's appended rows (the same
    inputs in both models) are the fp32-cache model's appended rows rounded
    to binary16, up to double rounding (one unit in the last place); every
    other slot of every layer is untouched; and the logits stay close to the
    fp32-cache model's."""
    from synth import workloads as wl
    m = wl.TINY_GEMMA4
    w = wl.model_weights(m)
    c32 = [(wl.prefilled_cache(m, l, "k").astype(np.float16).astype(np.float32),
            wl.prefilled_cache(m, l, "v").astype(np.float16).astype(np.float32))
           for l in range(m.n_layers)]
    c16 = [(k.astype(np.float16), v.astype(np.float16)) for k, v in c32]
    before = [(k.copy(), v.copy()) for k, v in c16]
    tok = wl.start_tokens(m)
    _, lg32, _ = oracle.Model(wl.oracle_spec(m, w, c32)).step(m.start_pos, tok, want_logits=True)
    _, lg16, _ = oracle.Model(wl.oracle_spec(m, w, c16)).step(m.start_pos, tok, want_logits=True)
    for l, ly in enumerate(m.layers):
        slot = m.start_pos % ly.cap
        for c in (0, 1):
            if l == 0:
                got = c16[l][c][:, :, slot].view(np.uint16).astype(np.int64)
                ref = c32[l][c][:, :, slot].astype(np.float16).view(np.uint16).astype(np.int64)
                assert np.all(np.abs(got - ref) <= 1) and np.mean(got == ref) > 0.99
            others = np.arange(ly.cap) != slot
            assert np.array_equal(c16[l][c][:, :, others], before[l][c][:, :, others])
    assert np.abs(lg16 - lg32).max() <= 1e-2 * np.abs(lg32).max()


# ---------------------------------------------------------------- Gemma-4 variants
def test_geglu_tanh_form():
    """GELU's tanh form: gelu(x) - gelu(-x) = x exactly (the form is x times an
    odd-symmetric sigmoid-like factor), zero at zero, within 1e-3 of the
    erf definition x Phi(x) everywhere (math.erf; a dropped cubic term misses
    by ~2e-2), and the up operand multiplies."""
    x = np.linspace(-6, 6, 2001)
    one = np.ones_like(x)
    g = oracle.geglu(x, one)
    assert np.allclose(g - oracle.geglu(-x, one), x, rtol=0, atol=1e-12)
    assert oracle.geglu(np.zeros(1), np.ones(1))[0] == 0.0
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    assert np.abs(g - exact).max() < 1e-3
    u = np.linspace(-2, 3, 2001)
    assert np.allclose(oracle.geglu(x, u), g * u, rtol=1e-15, atol=0)
    # large arguments: identity on the right, zero on the left
    assert abs(oracle.geglu(np.array([12.0]), np.ones(1))[0] - 12.0) < 1e-12
    assert abs(oracle.geglu(np.array([-12.0]), np.ones(1))[0]) < 1e-12


def test_softcap_properties():
    c = 30.0
    v = np.linspace(-500, 500, 4001)
    s = oracle.softcap(v, c)
    assert np.all(np.abs(s) <= c) and np.all(np.diff(s) >= 0)     # bounded, non-decreasing
    mid = oracle.softcap(np.linspace(-150, 150, 3001), c)
    assert np.all(np.abs(mid) < c) and np.all(np.diff(mid) > 0)  # strictly below saturation
    assert np.allclose(s, -oracle.softcap(-v, c), rtol=0, atol=1e-12)
    small = np.linspace(-0.3, 0.3, 101)
    assert np.allclose(oracle.softcap(small, c), small - small ** 3 / (3 * c * c), rtol=0, atol=1e-9)
    assert np.allclose(oracle.softcap(v, c), c * oracle.softcap(v / c, 1.0), rtol=1e-14, atol=1e-12)
    assert abs(oracle.softcap(np.array([1e6]), c)[0] - c) < 1e-12


def test_partial_rope_prefix_and_passthrough():
    """p-RoPE: the first r dims rotate exactly as a full NeoX rotation of the
    r-dim prefix (pinned above); the rest pass through; r = hd is full RoPE."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 512))
    for pos, r in ((0, 128), (77, 128), (8191, 128), (5, 64), (300, 512)):
        y = oracle.rope_neox(x, pos, 1e6, r)
        assert np.array_equal(y[:, r:], x[:, r:])
        assert np.allclose(y[:, :r], oracle.rope_neox(x[:, :r], pos, 1e6), rtol=0, atol=1e-15)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.array_equal(oracle.rope_neox(x, 9, 1e4, 512), oracle.rope_neox(x, 9, 1e4))
