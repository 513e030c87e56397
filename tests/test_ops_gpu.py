"""GPU parity of RMSNorm, SwiGLU, QK-norm + RoPE + KV append, GQA decode
attention and argmax against the fp64 oracle (element by element)."""
import math

import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
import synth
from q4_quantized_matvec_amd._lib import kv_layout_of

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("rows,dim,gain", [(1, 2560, True), (8, 5376, True), (3, 100, False),
                                           (5, 21504, True), (1, 1, True)])
def test_rmsnorm_parity(dev, rows, dim, gain):
    _say(f"rmsnorm {rows}x{dim} gain={gain}")
    x = synth.normal_f32(201, f"rms.x.{rows}.{dim}", (rows, dim)) * 3.0
    w = synth.uniform_f32(201, f"rms.w.{dim}", (dim,), 0.8, 1.2) if gain else None
    ref = oracle.rmsnorm(x, w, 1e-6)
    y = q.rmsnorm(torch.from_numpy(x).to(dev), None if w is None else torch.from_numpy(w).to(dev), 1e-6)
    torch.cuda.synchronize()
    err = np.abs(_np(y) - ref)
    assert np.all(err <= 2e-4 * np.abs(ref) + 1e-6)


def test_rmsnorm_in_place(dev):
    x = synth.normal_f32(202, "rms.inplace", (4, 2048))
    w = synth.uniform_f32(202, "rms.inplace.w", (2048,), 0.8, 1.2)
    ref = oracle.rmsnorm(x, w, 1e-6)
    xt = torch.from_numpy(x).to(dev)
    q.rmsnorm(xt, torch.from_numpy(w).to(dev), 1e-6, y=xt)
    torch.cuda.synchronize()
    assert np.all(np.abs(_np(xt) - ref) <= 2e-4 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("rows,n", [(1, 9728), (8, 9728), (3, 21504), (2, 7)])
def test_swiglu_parity_merged_rows(dev, rows, n):
    _say(f"swiglu {rows}x{n}")
    gu = synth.normal_f32(203, f"swiglu.{rows}.{n}", (rows, 2 * n)) * 4.0
    ref = np.stack([oracle.swiglu(gu[r, :n], gu[r, n:]) for r in range(rows)])
    g = torch.from_numpy(gu).to(dev)
    h = q.swiglu(g, g[:, n:], rows, n, 2 * n)
    torch.cuda.synchronize()
    assert np.all(np.abs(_np(h) - ref) <= 2e-4 * np.abs(ref) + 1e-6)


def _qk_case(dev, B, hq, hkv, hd, cap, pos, theta, v_from_k, seed, kv16=False):
    nq, nk = hq * hd, hkv * hd
    ld = nq + nk + (0 if v_from_k else nk)
    rows = synth.normal_f32(seed, f"qk.rows.{hd}.{pos}", (B, ld)) * 2.0
    qn = synth.uniform_f32(seed, f"qk.qn.{hd}", (hd,), 0.8, 1.2)
    kn = synth.uniform_f32(seed, f"qk.kn.{hd}", (hd,), 0.8, 1.2)
    kc = synth.normal_f32(seed, f"qk.kc.{hd}", (B, hkv, cap, hd))
    vc = synth.normal_f32(seed, f"qk.vc.{hd}", (B, hkv, cap, hd))
    if kv16:
        kc, vc = kc.astype(np.float16), vc.astype(np.float16)
    rows_d = torch.from_numpy(rows).to(dev)
    kc_d, vc_d = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    pos_d = torch.tensor([pos], dtype=torch.int64, device=dev)
    q.qk_norm_rope(rows_d, ld, rows_d[:, nq:], None if v_from_k else rows_d[:, nq + nk:], ld,
                   torch.from_numpy(qn).to(dev), torch.from_numpy(kn).to(dev), hq,
                   kv_layout_of(kc_d), pos_d, theta, 1e-6, v_from_k, kc_d, vc_d)
    torch.cuda.synchronize()
    return rows, qn, kn, kc, vc, _np(rows_d), _np(kc_d), _np(vc_d)


def _rope_tol(normed, pos, theta):
    """2e-4 * (|x_i cos| + |x_{i+h} sin|) + 1e-6 per output element."""
    hd = normed.shape[-1]
    h = hd // 2
    i = np.arange(h)
    ang = pos * theta ** (-(2.0 * i) / hd)
    c, s = np.abs(np.cos(ang)), np.abs(np.sin(ang))
    a, b = np.abs(normed[..., :h]), np.abs(normed[..., h:])
    t0 = a * c + b * s
    t1 = b * c + a * s
    return 2e-4 * np.concatenate([t0, t1], axis=-1) + 1e-6


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("pos,theta", [(0, 1e6), (7, 1e4), (4096, 1e6), (8200, 1e6)])
@pytest.mark.parametrize("v_from_k", [False, True])
def test_qk_norm_rope_parity(dev, hd, pos, theta, v_from_k):
    _say(f"qk_norm_rope hd={hd} pos={pos} theta={theta} v_from_k={v_from_k}")
    B, hq, hkv, cap = 2, 4, 2, 16
    rows, qn, kn, kc0, vc0, got, kc, vc = _qk_case(dev, B, hq, hkv, hd, cap, pos, theta,
                                                    v_from_k, 204)
    nq, nk = hq * hd, hkv * hd
    slot = pos % cap
    for b in range(B):
        qh = rows[b, :nq].reshape(hq, hd)
        kr = rows[b, nq:nq + nk].reshape(hkv, hd)
        qnorm = oracle.rmsnorm(qh, qn, 1e-6)
        qref = oracle.rope_neox(qnorm, pos, theta)
        assert np.all(np.abs(got[b, :nq].reshape(hq, hd) - qref) <= _rope_tol(qnorm, pos, theta))
        knorm = oracle.rmsnorm(kr, kn, 1e-6)
        kref = oracle.rope_neox(knorm, pos, theta)
        assert np.all(np.abs(kc[b, :, slot] - kref) <= _rope_tol(knorm, pos, theta))
        vref = (oracle.rmsnorm(kr, None, 1e-6) if v_from_k
                else rows[b, nq + nk:].reshape(hkv, hd).astype(np.float64))
        assert np.all(np.abs(vc[b, :, slot] - vref) <= 2e-4 * np.abs(vref) + 1e-6)
    # every other slot is untouched
    others = [s for s in range(cap) if s != slot]
    assert np.array_equal(kc[:, :, others], kc0[:, :, others])
    assert np.array_equal(vc[:, :, others], vc0[:, :, others])


def _attn_oracle(qh, kc, vc, n, window, scale, cap):
    """Visible positions of one sequence gathered in position order for the oracle."""
    hkv, _, hd = kc.shape
    keys = np.zeros((n, hkv, hd))
    vals = np.zeros((n, hkv, hd))
    lo = max(0, n - window) if window else 0
    lo = max(lo, n - cap)
    slots = np.arange(lo, n) % cap
    keys[lo:n] = kc[:, slots].transpose(1, 0, 2)
    vals[lo:n] = vc[:, slots].transpose(1, 0, 2)
    # positions below lo are never seen: the oracle window expresses the same set
    w = n - lo if (window or lo > 0) else 0
    return oracle.gqa_attention(qh, keys, vals, w, scale)


ATTN_CASES = [
    # (B, Hq, Hkv, hd, cap, n, window)
    (1, 16, 8, 128, 4097, 4097, 0),      # the 1.7B-shaped layer, full cache
    (3, 16, 8, 128, 300, 257, 0),        # ragged chunk tail
    (2, 32, 8, 128, 64, 1, 0),           # one key
    (1, 32, 16, 256, 1024, 1024, 1024),  # sliding window, full ring
    (1, 32, 16, 256, 1024, 3000, 1024),  # ring wrapped past capacity
    (1, 32, 4, 512, 600, 555, 0),        # 8:1 groups, head_dim 512
    (2, 16, 1, 64, 100, 77, 16),         # 16:1 groups, window smaller than n
    (1, 6, 6, 128, 50, 33, 0),           # multi-head (G = 1)
    (8, 32, 8, 128, 2064, 2049, 0),      # Qwen3-4B-shaped, B = 8
    # long contexts: 4096+ chunks in all, so one workgroup takes a split of
    # several 64-key chunks with a running softmax
    (1, 16, 8, 128, 32768, 32768, 0),    # 32K keys, every split full
    (1, 16, 8, 128, 40000, 33001, 0),    # ragged last split, empty splits past n
    (1, 16, 8, 128, 32768, 40000, 0),    # ring wrapped past capacity
    (4, 16, 8, 128, 8192, 8000, 0),      # B = 4
    (1, 16, 1, 64, 262144, 262000, 0),   # 16:1 groups, 256K keys
    (8, 16, 16, 64, 4096, 9000, 4096),   # sliding window over a wrapped ring
    (1, 32, 4, 512, 65552, 65536, 0),    # 31B full-layer shape at 64K keys
]


@pytest.mark.parametrize("B,hq,hkv,hd,cap,n,window", ATTN_CASES)
def test_gqa_decode_attn_parity(dev, B, hq, hkv, hd, cap, n, window):
    _say(f"gqa_decode_attn B={B} Hq={hq} Hkv={hkv} hd={hd} cap={cap} n={n} window={window}")
    seed = 205
    qv = synth.normal_f32(seed, f"att.q.{hd}.{hq}", (B, hq * hd))
    kc = synth.normal_f32(seed, f"att.k.{hd}.{cap}", (B, hkv, cap, hd))
    vc = synth.normal_f32(seed, f"att.v.{hd}.{cap}", (B, hkv, cap, hd))
    scale = 1.0 / math.sqrt(hd) if window == 0 else 1.0
    kc_d, vc_d = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    kv = kv_layout_of(kc_d)
    ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, window), dtype=torch.uint8, device=dev)
    out = torch.empty((B, hq * hd), dtype=torch.float32, device=dev)
    n_d = torch.tensor([n], dtype=torch.int64, device=dev)
    q.gqa_decode_attn(torch.from_numpy(qv).to(dev), hq * hd, hq, kc_d, vc_d, kv, n_d, window, scale,
                      out, hq * hd, ws)
    torch.cuda.synchronize()
    got = _np(out)
    worst = 0.0
    for b in range(B):
        o, bound = _attn_oracle(qv[b].reshape(hq, hd).astype(np.float64), kc[b].astype(np.float64),
                                vc[b].astype(np.float64), n, window, scale, cap)
        err = np.abs(got[b].reshape(hq, hd) - o)
        tol = 2e-4 * bound + 1e-6
        worst = max(worst, float((err / tol).max()))
    assert worst <= 1.0, f"max err/tol {worst:.3e}"


@pytest.mark.parametrize("B,cap", [(2, 3000), (1, 40000)], ids=["one_chunk_splits", "long"])
def test_gqa_decode_attn_deterministic(dev, B, cap):
    hq, hkv, hd = 16, 8, 128
    qv = torch.randn(B, hq * hd, device=dev)
    kc = torch.randn(B, hkv, cap, hd, device=dev)
    vc = torch.randn(B, hkv, cap, hd, device=dev)
    kv = kv_layout_of(kc)
    ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, 0), dtype=torch.uint8, device=dev)
    n_d = torch.tensor([cap - 1], dtype=torch.int64, device=dev)
    outs = []
    for _ in range(3):
        out = torch.empty((B, hq * hd), device=dev)
        q.gqa_decode_attn(qv, hq * hd, hq, kc, vc, kv, n_d, 0, 0.088, out, hq * hd, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_gqa_decode_attn_shared_workspace_mixed_shapes(dev):
    """One workspace shared by calls of different shapes, interleaved, as a
    decode step's layers share it: every call of a shape gives the same bits
    as its first call and as a call on a fresh workspace."""
    shapes = {"A": (1, 4, 2, 128, 512, 500), "B": (2, 16, 8, 128, 4096, 4000),
              "C": (1, 32, 4, 512, 1024, 1000)}
    gen = torch.Generator(device=dev)
    gen.manual_seed(207)
    ins = {}
    for key, (B, hq, hkv, hd, cap, n) in shapes.items():
        qv = torch.randn((B, hq * hd), device=dev, generator=gen)
        kc = torch.randn((B, hkv, cap, hd), device=dev, generator=gen)
        vc = torch.randn((B, hkv, cap, hd), device=dev, generator=gen)
        ins[key] = (qv, kc, vc, kv_layout_of(kc), torch.tensor([n], dtype=torch.int64, device=dev),
                    hq, hd)
    size = max(q.gqa_decode_attn_workspace(v[3], v[5], 0) for v in ins.values())
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)

    def run(key, wsp):
        qv, kc, vc, kv, n_d, hq, hd = ins[key]
        out = torch.empty((qv.shape[0], hq * hd), device=dev)
        q.gqa_decode_attn(qv, hq * hd, hq, kc, vc, kv, n_d, 0, 1.0 / math.sqrt(hd), out, hq * hd, wsp)
        return out

    first = {}
    for key in "ABCACBA":
        out = run(key, ws)
        if key in first:
            assert torch.equal(out, first[key]), f"shape {key} changed on a shared workspace"
        else:
            first[key] = out
    for key in "ABC":
        fresh = torch.zeros(q.gqa_decode_attn_workspace(ins[key][3], ins[key][5], 0), dtype=torch.uint8,
                            device=dev)
        assert torch.equal(run(key, fresh), first[key])
    torch.cuda.synchronize()


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "two_pass"])
def test_argmax_rows_ties_and_parity(dev, two_pass):
    _say(f"argmax_rows two_pass={two_pass}")
    V = 262144
    lg = synth.normal_f32(206, "argmax", (6, V)) * 10.0
    lg[1, 100] = lg[1, 7] = lg[1].max() + 1.0   # tie: lowest id wins
    lg[2, :] = -np.inf
    lg[3, 5] = np.nan
    lg[3, 9] = 1e30
    # a tie across the two-pass slices (4096 columns each) and a row maximum
    # in the last, partial position
    lg[4, 5000] = lg[4, 200000] = lg[4].max() + 1.0
    lg[5, V - 1] = lg[5].max() + 1.0
    fn = q.argmax_rows_ws if two_pass else q.argmax_rows
    got = fn(torch.from_numpy(lg).to(dev)).cpu().numpy()
    exp = [oracle.argmax(lg[0])[0], 7, 0, 9, 5000, V - 1]
    assert got.tolist() == exp
    if two_pass:  # odd vocabulary sizes, shorter than the slice count, B = 1..3
        for v_, b_ in ((151936, 3), (1000, 2), (37, 1)):
            x = synth.normal_f32(207, f"argmax.{v_}", (b_, v_))
            g = q.argmax_rows_ws(torch.from_numpy(x).to(dev)).cpu().numpy()
            assert g.tolist() == [oracle.argmax(x[i])[0] for i in range(b_)]


ROPE_ATTN_CASES = [
    # (B, Hq, Hkv, hd, cap, pos, window, v_from_k, theta); n = pos + 1
    (1, 16, 8, 128, 4097, 4096, 0, False, 1e6),   # the 1.7B-shaped layer
    (3, 16, 8, 128, 300, 256, 0, False, 1e6),     # ragged chunk tail
    (2, 32, 8, 128, 64, 0, 0, False, 1e6),        # the new key is the only key
    (1, 32, 16, 256, 1024, 3000, 1024, False, 1e4),  # sliding window, wrapped ring
    (1, 32, 4, 512, 8208, 8192, 0, True, 1e6),    # 31B full layer: V from K
    (2, 16, 1, 64, 100, 76, 16, True, 1e4),       # 16:1 groups, small window
    (8, 32, 8, 128, 2064, 2048, 0, False, 1e6),   # 4B-shaped, B = 8
    # long contexts (splits of several chunks; the append lands in the last)
    (1, 32, 4, 512, 65552, 65536, 0, True, 1e6),  # 31B full layer at 64K keys
    (1, 16, 8, 128, 32768, 40000, 0, False, 1e6),  # wrapped ring
]


@pytest.mark.parametrize("B,hq,hkv,hd,cap,pos,window,v_from_k,theta", ROPE_ATTN_CASES)
def test_gqa_decode_attn_rope_parity(dev, B, hq, hkv, hd, cap, pos, window, v_from_k, theta):
    """Fused QK-norm + RoPE + KV append + attention against the oracle ops."""
    _say(f"gqa_decode_attn_rope B={B} Hq={hq} Hkv={hkv} hd={hd} cap={cap} pos={pos} "
         f"window={window} v_from_k={v_from_k}")
    seed = 206
    nq, nk = hq * hd, hkv * hd
    ld = nq + nk + (0 if v_from_k else nk)
    rows = synth.normal_f32(seed, f"ra.rows.{hd}.{pos}", (B, ld)) * 2.0
    qn = synth.uniform_f32(seed, f"ra.qn.{hd}", (hd,), 0.8, 1.2)
    kn = synth.uniform_f32(seed, f"ra.kn.{hd}", (hd,), 0.8, 1.2)
    kc0 = synth.normal_f32(seed, f"ra.kc.{hd}.{cap}", (B, hkv, cap, hd))
    vc0 = synth.normal_f32(seed, f"ra.vc.{hd}.{cap}", (B, hkv, cap, hd))
    scale = 1.0 / math.sqrt(hd) if not v_from_k else 1.0
    kc_d, vc_d = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
    kv = kv_layout_of(kc_d)
    ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, window), dtype=torch.uint8, device=dev)
    out = torch.empty((B, nq), dtype=torch.float32, device=dev)
    pos_d = torch.tensor([pos], dtype=torch.int64, device=dev)
    q.gqa_decode_attn_rope(torch.from_numpy(rows).to(dev), ld, hq, torch.from_numpy(qn).to(dev),
                           torch.from_numpy(kn).to(dev), kv, pos_d, theta, 1e-6, v_from_k, kc_d, vc_d,
                           window, scale, out, nq, ws)
    torch.cuda.synchronize()
    kc, vc, got = _np(kc_d), _np(vc_d), _np(out)
    slot = pos % cap
    others = np.arange(cap) != slot
    assert np.array_equal(kc[:, :, others], kc0[:, :, others])
    assert np.array_equal(vc[:, :, others], vc0[:, :, others])
    worst = 0.0
    for b in range(B):
        kr = rows[b, nq:nq + nk].reshape(hkv, hd)
        knorm = oracle.rmsnorm(kr, kn, 1e-6)
        kref = oracle.rope_neox(knorm, pos, theta)
        assert np.all(np.abs(kc[b, :, slot] - kref) <= _rope_tol(knorm, pos, theta))
        vref = (oracle.rmsnorm(kr, None, 1e-6) if v_from_k
                else rows[b, nq + nk:].reshape(hkv, hd).astype(np.float64))
        assert np.all(np.abs(vc[b, :, slot] - vref) <= 2e-4 * np.abs(vref) + 1e-6)
        qref = oracle.rope_neox(oracle.rmsnorm(rows[b, :nq].reshape(hq, hd), qn, 1e-6), pos, theta)
        o, bound = _attn_oracle(qref, kc[b].astype(np.float64), vc[b].astype(np.float64), pos + 1,
                                window, scale, cap)
        err = np.abs(got[b].reshape(hq, hd) - o)
        worst = max(worst, float((err / (2e-4 * bound + 1e-6)).max()))
    assert worst <= 1.0, f"max err/tol {worst:.3e}"


# ---------------------------------------------------------------- binary16 KV caches
# Cached elements are read exactly (the oracle gets the same binary16 values
# as fp64); appended rows are computed in fp32 and rounded to the nearest
# binary16, so their bound adds half a unit in the last place, 2^-11 |x|.
F16_ULP = 2.0 ** -11


@pytest.mark.parametrize("hd", [128, 512])
@pytest.mark.parametrize("pos,theta", [(7, 1e4), (8200, 1e6)])
@pytest.mark.parametrize("v_from_k", [False, True])
def test_qk_norm_rope_f16_cache(dev, hd, pos, theta, v_from_k):
    _say(f"qk_norm_rope f16 cache hd={hd} pos={pos} v_from_k={v_from_k}")
    B, hq, hkv, cap = 2, 4, 2, 16
    rows, qn, kn, kc0, vc0, got, kc, vc = _qk_case(dev, B, hq, hkv, hd, cap, pos, theta,
                                                    v_from_k, 214, kv16=True)
    nq, nk = hq * hd, hkv * hd
    slot = pos % cap
    for b in range(B):
        qnorm = oracle.rmsnorm(rows[b, :nq].reshape(hq, hd), qn, 1e-6)
        qref = oracle.rope_neox(qnorm, pos, theta)
        assert np.all(np.abs(got[b, :nq].reshape(hq, hd) - qref) <= _rope_tol(qnorm, pos, theta))
        kr = rows[b, nq:nq + nk].reshape(hkv, hd)
        knorm = oracle.rmsnorm(kr, kn, 1e-6)
        kref = oracle.rope_neox(knorm, pos, theta)
        assert np.all(np.abs(kc[b, :, slot] - kref) <= _rope_tol(knorm, pos, theta) +
                      F16_ULP * np.abs(kref))
        vref = (oracle.rmsnorm(kr, None, 1e-6) if v_from_k
                else rows[b, nq + nk:].reshape(hkv, hd).astype(np.float64))
        assert np.all(np.abs(vc[b, :, slot] - vref) <= (2e-4 + F16_ULP) * np.abs(vref) + 1e-6)
    others = np.arange(cap) != slot
    assert np.array_equal(kc[:, :, others], kc0[:, :, others].astype(np.float64))
    assert np.array_equal(vc[:, :, others], vc0[:, :, others].astype(np.float64))


F16_ATTN_CASES = [
    # (B, Hq, Hkv, hd, cap, n, window)
    (1, 16, 8, 128, 4097, 4097, 0),      # the 1.7B-shaped layer
    (3, 16, 8, 128, 300, 257, 0),        # ragged chunk tail
    (1, 32, 16, 256, 1024, 3000, 1024),  # sliding window, wrapped ring
    (1, 32, 4, 512, 8208, 8193, 0),      # 31B full layer
    (8, 32, 8, 128, 2064, 2049, 0),      # Qwen3-4B-shaped, B = 8
    (1, 16, 8, 128, 40000, 33001, 0),    # multi-chunk splits, ragged
    (1, 32, 4, 512, 65552, 65536, 0),    # 31B full layer at 64K keys
    (2, 28, 4, 512, 700, 650, 0),        # hd 512, 7:1 groups, B = 2, ragged tail
    (1, 32, 4, 512, 1024, 3000, 1024),   # hd 512, sliding window, wrapped ring
    (1, 64, 8, 128, 600, 555, 0),        # hd 128, 8:1 groups
    (2, 24, 8, 128, 500, 450, 0),        # hd 128, 3:1 groups (a zero operand row pair)
    (1, 48, 16, 256, 900, 777, 0),       # hd 256, 3:1 groups
]


@pytest.mark.parametrize("B,hq,hkv,hd,cap,n,window", F16_ATTN_CASES)
def test_gqa_decode_attn_f16_cache_parity(dev, B, hq, hkv, hd, cap, n, window):
    _say(f"gqa_decode_attn f16 cache B={B} Hq={hq} Hkv={hkv} hd={hd} cap={cap} n={n}")
    seed = 215
    qv = synth.normal_f32(seed, f"att16.q.{hd}.{hq}", (B, hq * hd))
    kc = synth.normal_f32(seed, f"att16.k.{hd}.{cap}", (B, hkv, cap, hd)).astype(np.float16)
    vc = synth.normal_f32(seed, f"att16.v.{hd}.{cap}", (B, hkv, cap, hd)).astype(np.float16)
    scale = 1.0 / math.sqrt(hd) if window == 0 else 1.0
    kc_d, vc_d = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    kv = kv_layout_of(kc_d)
    assert kv.dtype == 1
    ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, window), dtype=torch.uint8, device=dev)
    out = torch.empty((B, hq * hd), dtype=torch.float32, device=dev)
    n_d = torch.tensor([n], dtype=torch.int64, device=dev)
    q.gqa_decode_attn(torch.from_numpy(qv).to(dev), hq * hd, hq, kc_d, vc_d, kv, n_d, window, scale,
                      out, hq * hd, ws)
    torch.cuda.synchronize()
    got = _np(out)
    worst = 0.0
    for b in range(B):
        o, bound = _attn_oracle(qv[b].reshape(hq, hd).astype(np.float64), kc[b].astype(np.float64),
                                vc[b].astype(np.float64), n, window, scale, cap)
        worst = max(worst, float((np.abs(got[b].reshape(hq, hd) - o) / (2e-4 * bound + 1e-6)).max()))
    assert worst <= 1.0, f"max err/tol {worst:.3e}"


@pytest.mark.parametrize("B,hq,hkv,hd,cap,pos,window,v_from_k,theta", [
    (1, 16, 8, 128, 4097, 4096, 0, False, 1e6),
    (1, 32, 16, 256, 1024, 3000, 1024, False, 1e4),
    (1, 32, 4, 512, 8208, 8192, 0, True, 1e6),
    (8, 32, 8, 128, 2064, 2048, 0, False, 1e6),
    (1, 32, 4, 512, 65552, 65536, 0, True, 1e6),
    (2, 28, 4, 512, 700, 640, 0, False, 1e6),
])
def test_gqa_decode_attn_rope_f16_cache(dev, B, hq, hkv, hd, cap, pos, window, v_from_k, theta):
    """Fused preparation, binary16 append and attention over binary16 caches."""
    _say(f"gqa_decode_attn_rope f16 cache B={B} Hq={hq} Hkv={hkv} hd={hd} cap={cap} pos={pos}")
    seed = 216
    nq, nk = hq * hd, hkv * hd
    ld = nq + nk + (0 if v_from_k else nk)
    rows = synth.normal_f32(seed, f"ra16.rows.{hd}.{pos}", (B, ld)) * 2.0
    qn = synth.uniform_f32(seed, f"ra16.qn.{hd}", (hd,), 0.8, 1.2)
    kn = synth.uniform_f32(seed, f"ra16.kn.{hd}", (hd,), 0.8, 1.2)
    kc0 = synth.normal_f32(seed, f"ra16.kc.{hd}.{cap}", (B, hkv, cap, hd)).astype(np.float16)
    vc0 = synth.normal_f32(seed, f"ra16.vc.{hd}.{cap}", (B, hkv, cap, hd)).astype(np.float16)
    scale = 1.0 / math.sqrt(hd) if not v_from_k else 1.0
    kc_d, vc_d = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
    kv = kv_layout_of(kc_d)
    ws = torch.zeros(q.gqa_decode_attn_workspace(kv, hq, window), dtype=torch.uint8, device=dev)
    out = torch.empty((B, nq), dtype=torch.float32, device=dev)
    pos_d = torch.tensor([pos], dtype=torch.int64, device=dev)
    q.gqa_decode_attn_rope(torch.from_numpy(rows).to(dev), ld, hq, torch.from_numpy(qn).to(dev),
                           torch.from_numpy(kn).to(dev), kv, pos_d, theta, 1e-6, v_from_k, kc_d, vc_d,
                           window, scale, out, nq, ws)
    torch.cuda.synchronize()
    kc, vc, got = _np(kc_d), _np(vc_d), _np(out)
    slot = pos % cap
    others = np.arange(cap) != slot
    assert np.array_equal(kc[:, :, others], kc0[:, :, others].astype(np.float64))
    assert np.array_equal(vc[:, :, others], vc0[:, :, others].astype(np.float64))
    worst = 0.0
    for b in range(B):
        kr = rows[b, nq:nq + nk].reshape(hkv, hd)
        knorm = oracle.rmsnorm(kr, kn, 1e-6)
        kref = oracle.rope_neox(knorm, pos, theta)
        assert np.all(np.abs(kc[b, :, slot] - kref) <= _rope_tol(knorm, pos, theta) +
                      F16_ULP * np.abs(kref))
        vref = (oracle.rmsnorm(kr, None, 1e-6) if v_from_k
                else rows[b, nq + nk:].reshape(hkv, hd).astype(np.float64))
        assert np.all(np.abs(vc[b, :, slot] - vref) <= (2e-4 + F16_ULP) * np.abs(vref) + 1e-6)
        qref = oracle.rope_neox(oracle.rmsnorm(rows[b, :nq].reshape(hq, hd), qn, 1e-6), pos, theta)
        o, bound = _attn_oracle(qref, kc[b], vc[b], pos + 1, window, scale, cap)
        worst = max(worst, float((np.abs(got[b].reshape(hq, hd) - o) / (2e-4 * bound + 1e-6)).max()))
    assert worst <= 1.0, f"max err/tol {worst:.3e}"


# ---------------------------------------------------------------- Gemma-4 variants
@pytest.mark.parametrize("rows,n", [(1, 21504), (8, 9728), (3, 7)])
def test_geglu_parity(dev, rows, n):
    _say(f"geglu {rows}x{n}")
    gu = synth.normal_f32(217, f"geglu.{rows}.{n}", (rows, 2 * n)) * 4.0
    ref = np.stack([oracle.geglu(gu[r, :n], gu[r, n:]) for r in range(rows)])
    g = torch.from_numpy(gu).to(dev)
    h = q.geglu(g, g[:, n:], rows, n, 2 * n)
    torch.cuda.synchronize()
    assert np.all(np.abs(_np(h) - ref) <= 2e-4 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("rows,dim,gain", [(1, 5376, True), (8, 2560, True), (3, 100, False)])
def test_rmsnorm_add_parity(dev, rows, dim, gain):
    """x += w * y / rms(y): the sandwich post-norm joining the residual."""
    _say(f"rmsnorm_add {rows}x{dim}")
    y = synth.normal_f32(218, f"rna.y.{rows}.{dim}", (rows, dim)) * 3.0
    x0 = synth.normal_f32(218, f"rna.x.{rows}.{dim}", (rows, dim))
    w = synth.uniform_f32(218, f"rna.w.{dim}", (dim,), 0.8, 1.2) if gain else None
    normed = oracle.rmsnorm(y, w, 1e-6)
    ref = x0.astype(np.float64) + normed
    xd = torch.from_numpy(x0).to(dev)
    q.rmsnorm_add(torch.from_numpy(y).to(dev), torch.from_numpy(w).to(dev) if gain else None, 1e-6, xd)
    torch.cuda.synchronize()
    assert np.all(np.abs(_np(xd) - ref) <= 2e-4 * np.abs(normed) + 2.0 ** -23 * np.abs(ref) + 1e-6)


def test_softcap_parity(dev):
    _say("softcap")
    v = synth.normal_f32(219, "softcap", (4, 262144)) * 40.0
    ref = oracle.softcap(v, 30.0)
    vd = torch.from_numpy(v).to(dev)
    q.softcap(vd, 30.0)
    torch.cuda.synchronize()
    got = _np(vd)
    assert np.all(np.abs(got - ref) <= 2e-6 * 30.0)
    # increasing: the greedy choice is the same before and after
    assert np.array_equal(got.argmax(axis=1), v.argmax(axis=1))


@pytest.mark.parametrize("hd,rot", [(512, 128), (256, 64), (128, 32), (64, 16), (128, 128)])
@pytest.mark.parametrize("v_from_k", [False, True])
def test_qk_norm_rope_partial_parity(dev, hd, rot, v_from_k):
    """p-RoPE: the first rot elements rotate (as a rot-dim NeoX rotation), the
    rest are only normalised; q in place, k and v appended."""
    _say(f"qk_norm_rope_partial hd={hd} rot={rot} v_from_k={v_from_k}")
    B, hq, hkv, cap, pos, theta = 2, 4, 2, 16, 8200, 1e6
    nq, nk = hq * hd, hkv * hd
    ld = nq + nk + (0 if v_from_k else nk)
    rows = synth.normal_f32(220, f"qkp.rows.{hd}", (B, ld)) * 2.0
    qn = synth.uniform_f32(220, f"qkp.qn.{hd}", (hd,), 0.8, 1.2)
    kn = synth.uniform_f32(220, f"qkp.kn.{hd}", (hd,), 0.8, 1.2)
    kc0 = synth.normal_f32(220, f"qkp.kc.{hd}", (B, hkv, cap, hd))
    vc0 = synth.normal_f32(220, f"qkp.vc.{hd}", (B, hkv, cap, hd))
    rows_d = torch.from_numpy(rows).to(dev)
    kc_d, vc_d = torch.from_numpy(kc0).to(dev), torch.from_numpy(vc0).to(dev)
    pos_d = torch.tensor([pos], dtype=torch.int64, device=dev)
    q.qk_norm_rope(rows_d, ld, rows_d[:, nq:], None if v_from_k else rows_d[:, nq + nk:], ld,
                   torch.from_numpy(qn).to(dev), torch.from_numpy(kn).to(dev), hq,
                   kv_layout_of(kc_d), pos_d, theta, 1e-6, v_from_k, kc_d, vc_d, rot_dims=rot)
    torch.cuda.synchronize()
    got, kc, vc = _np(rows_d), _np(kc_d), _np(vc_d)
    slot = pos % cap

    def tol(normed):
        t = np.concatenate([_rope_tol(normed[..., :rot], pos, theta),
                            2e-4 * np.abs(normed[..., rot:]) + 1e-6], axis=-1)
        return t

    for b in range(B):
        qnorm = oracle.rmsnorm(rows[b, :nq].reshape(hq, hd), qn, 1e-6)
        qref = oracle.rope_neox(qnorm, pos, theta, rot)
        assert np.all(np.abs(got[b, :nq].reshape(hq, hd) - qref) <= tol(qnorm))
        kr = rows[b, nq:nq + nk].reshape(hkv, hd)
        knorm = oracle.rmsnorm(kr, kn, 1e-6)
        kref = oracle.rope_neox(knorm, pos, theta, rot)
        assert np.all(np.abs(kc[b, :, slot] - kref) <= tol(knorm))
        vref = (oracle.rmsnorm(kr, None, 1e-6) if v_from_k
                else rows[b, nq + nk:].reshape(hkv, hd).astype(np.float64))
        assert np.all(np.abs(vc[b, :, slot] - vref) <= 2e-4 * np.abs(vref) + 1e-6)
    others = np.arange(cap) != slot
    assert np.array_equal(kc[:, :, others], kc0[:, :, others])
