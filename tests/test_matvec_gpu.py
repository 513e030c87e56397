"""GPU parity of the Q4_0 / Q8_0 matvec and the Q8_0 gather against the oracle.

Bar: |gpu - oracle| <= 2e-4 * sum_k |w_k x_k| (+ |residual|) + 1e-6 per output.
"""
import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
import synth
from synth import workloads as wl

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(y, ref, terms, what):
    y = y.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
    err = np.abs(y - ref)
    tol = 2e-4 * terms + 1e-6
    ratio = float((err / tol).max())
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert ratio <= 1.0, f"{what}: max err/tol {ratio:.3e}"
    return ratio


CASES_Q4 = [
    # (N, K, B): fast path (B=1, K%256==0) incl. every register/K-split variant,
    # ragged row tails, and the generic path (K%256 != 0 or B > 1)
    (67, 256, 1), (1, 256, 1), (5, 2048, 1), (1000, 2048, 1), (777, 5376, 1), (300, 8192, 1),
    (200, 16384, 1), (130, 21504, 1), (257, 2560, 1), (99, 9728, 1),
    (67, 32, 1), (67, 288, 3), (33, 256, 8), (100, 2560, 8), (64, 5376, 2), (50, 9728, 4),
    # B > 1 on the vector kernel (one weight pass per batch row) at every K split
    (300, 8192, 3), (129, 16384, 2), (1000, 2048, 5), (77, 5376, 7), (200, 21504, 6), (90, 256, 2),
    # 3 <= B <= 8 with many rows: the matrix-core tile kernel over the whole K
    # (no workspace), ragged row tails
    (16390, 2560, 3), (4100, 1024, 6), (5000, 2048, 8), (16400, 256, 4),
]


@pytest.mark.parametrize("n,k,b", CASES_Q4)
def test_q4_0_matvec_parity(dev, n, k, b):
    _say(f"q4_0_matvec N={n} K={k} B={b}")
    W = synth.q4_0_matrix(101, f"t.q4.{n}.{k}", n, k)
    x = synth.normal_f32(101, f"t.q4x.{n}.{k}.{b}", (b, k))
    ref, terms = oracle.q4_0_matvec(W, n, k, x)
    y = q.q4_0_matvec(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    _check(y, ref, terms, f"q4 {n}x{k} B={b}")


@pytest.mark.parametrize("n,k,b", [(67, 256, 1), (1000, 2560, 1), (500, 5376, 1),
                                   (100, 2560, 8), (31, 32, 1), (300, 21504, 1), (40, 288, 5),
                                   (16400, 2560, 4), (4099, 1024, 7)])
def test_q8_0_matvec_parity(dev, n, k, b):
    _say(f"q8_0_matvec N={n} K={k} B={b}")
    W = synth.q8_0_matrix(102, f"t.q8.{n}.{k}", n, k)
    x = synth.normal_f32(102, f"t.q8x.{n}.{k}.{b}", (b, k))
    ref, terms = oracle.q8_0_matvec(W, n, k, x)
    y = q.q8_0_matvec(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    _check(y, ref, terms, f"q8 {n}x{k} B={b}")


@pytest.mark.parametrize("fmt", ["q4", "q8"])
@pytest.mark.parametrize("b,n", [(1, 513), (3, 513), (3, 16400)])
def test_matvec_residual_in_place(dev, fmt, b, n):
    _say(f"{fmt} residual in place B={b} N={n}")
    k = 2048
    gen = synth.q4_0_matrix if fmt == "q4" else synth.q8_0_matrix
    orc = oracle.q4_0_matvec if fmt == "q4" else oracle.q8_0_matvec
    fn = q.q4_0_matvec if fmt == "q4" else q.q8_0_matvec
    W = gen(103, f"t.res.{fmt}", n, k)
    x = synth.normal_f32(103, f"t.resx.{b}", (b, k))
    r = synth.normal_f32(103, f"t.resr.{b}", (b, n))
    ref, terms = orc(W, n, k, x, res=r)
    yr = torch.from_numpy(r).to(dev)
    fn(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev), y=yr, residual=yr)
    torch.cuda.synchronize()
    _check(yr, ref, terms, f"{fmt} residual alias")


@pytest.mark.parametrize("b", [1, 8])
def test_matvec_5376x21504_full(dev, b):
    """The 31B FFN-shape workload, every output, in the launch configuration the
    benchmark times."""
    _say(f"q4_0_matvec 5376x21504 B={b} full")
    w = wl.MATVEC_5376x21504
    W, x = wl.matvec_inputs(w, b)
    ref, terms = oracle.q4_0_matvec(W, w.n, w.k, x)
    Wd = torch.from_numpy(W).to(dev)
    xd = torch.from_numpy(x).to(dev)
    y1 = q.q4_0_matvec(Wd, xd)
    y2 = q.q4_0_matvec(Wd, xd)
    torch.cuda.synchronize()
    _check(y1, ref, terms, f"5376x21504 B={b}")
    assert torch.equal(y1, y2), "repeated launches differ bitwise"


def test_matvec_2048x6144_full(dev):
    _say("q4_0_matvec 2048x6144 B=1 full")
    w = wl.MATVEC_2048x6144
    W, x = wl.matvec_inputs(w, 1)
    ref, terms = oracle.q4_0_matvec(W, w.n, w.k, x)
    y = q.q4_0_matvec(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    _check(y, ref, terms, "2048x6144")


def test_q8_0_gather_parity(dev):
    _say("q8_0_gather")
    v, k = 1000, 2560
    E = synth.q8_0_matrix(104, "t.gather", v, k)
    tok = np.array([0, 999, 17, 17, 512], dtype=np.int32)
    ref = oracle.q8_0_gather(E, v, k, tok)
    x = q.q8_0_gather(torch.from_numpy(E).to(dev), torch.from_numpy(tok).to(dev), k)
    torch.cuda.synchronize()
    got = x.cpu().numpy().astype(np.float64)
    # d * q is exact in fp32 (11-bit scale times 8-bit code)
    assert np.array_equal(got, ref)


def test_q8_0_gather_out_of_range_token_gives_nan(dev):
    _say("q8_0_gather out-of-range")
    v, k = 50, 64
    E = synth.q8_0_matrix(105, "t.gather2", v, k)
    tok = torch.tensor([3, -1, 50], dtype=torch.int32, device=dev)
    x = q.q8_0_gather(torch.from_numpy(E).to(dev), tok, k)
    torch.cuda.synchronize()
    x = x.cpu().numpy()
    assert np.all(np.isfinite(x[0])) and np.all(np.isnan(x[1])) and np.all(np.isnan(x[2]))


FUSED_CASES = [
    # (fmt, N, K, B, op): LDS-staged (K <= 8192), split-K (K = 21504) and B > 1 paths
    ("q4", 300, 2560, 1, "rms"), ("q4", 257, 5376, 1, "swiglu"), ("q4", 200, 21504, 1, "swiglu"),
    ("q4", 130, 21504, 1, "rms"), ("q4", 100, 2560, 8, "rms"), ("q4", 64, 9728, 8, "swiglu"),
    ("q8", 1000, 5376, 1, "rms"), ("q8", 300, 2560, 8, "rms"), ("q4", 77, 2048, 1, "rms_unit"),
    # GeGLU input (tanh-form GELU gate): LDS-staged, split-K, B > 1
    ("q4", 257, 5376, 1, "geglu"), ("q4", 200, 21504, 1, "geglu"), ("q4", 64, 9728, 8, "geglu"),
    # B > 1 on the vector kernel with each input transform
    ("q4", 300, 5376, 3, "rms"), ("q4", 129, 8192, 2, "swiglu"), ("q4", 500, 2560, 4, "geglu"),
    ("q8", 200, 5376, 6, "rms_unit"),
    # ... and on the matrix-core tile kernel over the whole K (many rows)
    ("q4", 16390, 2560, 4, "rms"), ("q4", 8200, 2048, 7, "swiglu"), ("q4", 4100, 1024, 6, "geglu"),
    ("q8", 16400, 2560, 3, "rms"), ("q4", 5000, 2048, 8, "rms_unit"),
    # activation rows with a stride past K
    ("q4", 16390, 2560, 4, "rms_strided"), ("q4", 300, 5376, 1, "rms_strided"),
    ("q4", 5000, 2048, 7, "plain_strided"), ("q4", 200, 21504, 2, "plain_strided"),
]


@pytest.mark.parametrize("fmt,n,k,b,op", FUSED_CASES)
def test_matvec_fused_input_parity(dev, fmt, n, k, b, op):
    _say(f"{fmt} fused {op} N={n} K={k} B={b}")
    gen = synth.q4_0_matrix if fmt == "q4" else synth.q8_0_matrix
    orc = oracle.q4_0_matvec if fmt == "q4" else oracle.q8_0_matvec
    fn = q.q4_0_matvec_fused if fmt == "q4" else q.q8_0_matvec_fused
    W = gen(106, f"t.fused.{fmt}.{n}.{k}", n, k)
    ld = 2 * k if op in ("swiglu", "geglu") else k + 64 if op.endswith("_strided") else k
    xa = synth.normal_f32(106, f"t.fused.x.{k}.{b}", (b, ld)) * 2.0
    w = synth.uniform_f32(106, f"t.fused.w.{k}", (k,), 0.8, 1.2)
    r = synth.normal_f32(106, f"t.fused.r.{n}.{b}", (b, n))
    if op == "swiglu":
        xin = np.stack([oracle.swiglu(xa[i, :k], xa[i, k:]) for i in range(b)])
    elif op == "geglu":
        xin = np.stack([oracle.geglu(xa[i, :k], xa[i, k:]) for i in range(b)])
    elif op == "plain_strided":
        xin = xa[:, :k].astype(np.float64)
    else:
        xin = oracle.rmsnorm(xa[:, :k], None if op == "rms_unit" else w, 1e-6)
    ref, terms = orc(W, n, k, xin, res=r)
    xd = torch.from_numpy(xa).to(dev)
    yr = torch.from_numpy(r).to(dev)
    kind = {"swiglu": q.IN_SWIGLU, "geglu": q.IN_GEGLU, "plain_strided": q.IN_PLAIN}.get(op, q.IN_RMSNORM)
    fn(torch.from_numpy(W).to(dev), xd, k, b, ld, kind,
       x2=xd[:, k:] if op in ("swiglu", "geglu") else None,
       norm_w=torch.from_numpy(w).to(dev) if op in ("rms", "rms_strided") else None, eps=1e-6, y=yr,
       residual=yr)
    torch.cuda.synchronize()
    _check(yr, ref, terms, f"{fmt} fused {op} {n}x{k} B={b}")


BATCHED_CASES = [
    # (fmt, N, K, B, op): one split (S = 1) and K split over workgroups (S > 1),
    # ragged row tails, every batch count, each input transform
    ("q4", 67, 256, 2, "plain"), ("q4", 16, 256, 1, "plain"), ("q4", 1000, 2560, 8, "rms"),
    ("q4", 300, 9728, 8, "swiglu"), ("q4", 2560, 4096, 8, "plain"), ("q4", 777, 5376, 3, "plain"),
    ("q4", 33, 512, 5, "rms_unit"), ("q4", 6144, 2560, 8, "rms"), ("q4", 130, 21504, 7, "swiglu"),
    ("q8", 500, 2560, 8, "rms"), ("q8", 100, 256, 4, "plain"), ("q8", 3001, 2560, 6, "plain"),
    # shapes large enough for the tile kernel (each wavefront converts its own
    # step for several row tiles): every transform, Q8_0, ragged rows, B < 8,
    # with and without a K split, and two rounds per wavefront (K > 32768)
    ("q4", 8200, 4096, 8, "rms"), ("q4", 8192, 4096, 3, "swiglu"), ("q4", 33000, 1024, 5, "plain"),
    ("q4", 2000, 33024, 2, "rms"), ("q8", 8200, 2048, 8, "rms"), ("q8", 16400, 1024, 2, "plain"),
    # more than 8 rows: groups of 8 (the last one ragged), small and large
    # shapes, every transform, and more row ranges x groups than split tickets
    ("q4", 2000, 2560, 9, "rms"), ("q4", 2560, 4096, 16, "plain"), ("q4", 300, 9728, 13, "swiglu"),
    ("q4", 8192, 4096, 32, "swiglu"), ("q4", 8200, 4096, 24, "rms"), ("q4", 33000, 1024, 17, "plain"),
    ("q8", 8200, 2048, 20, "rms"), ("q8", 3001, 2560, 32, "plain"), ("q8", 140000, 256, 12, "rms"),
    # GeGLU input on both kernels
    ("q4", 300, 9728, 8, "geglu"), ("q4", 8192, 4096, 16, "geglu"), ("q4", 130, 21504, 3, "geglu"),
    # the K-stationary kernel: whole K per workgroup (K <= 12 steps, idle
    # wavefronts past the last step) and K ranges of 4 steps added by the
    # second launch (13 steps: the last range has one live wavefront), ragged
    # rows, one and several batch groups, every transform
    ("q4", 4100, 2560, 8, "rms"), ("q4", 16390, 3328, 8, "rms"), ("q4", 16390, 3328, 12, "swiglu"),
    ("q4", 8193, 5376, 1, "plain"), ("q4", 12000, 768, 20, "rms_unit"), ("q4", 8200, 5376, 6, "geglu"),
    # ... with 2 to 4 batch groups: whole K with 12, 8 and 4 wavefronts, K
    # ranges added by the second launch, a ragged last group, every transform
    ("q4", 6144, 2560, 16, "rms"), ("q4", 5000, 2048, 29, "plain"), ("q4", 4100, 1024, 32, "rms"),
    ("q4", 8200, 5376, 10, "plain"), ("q4", 8200, 3328, 16, "geglu"), ("q4", 16390, 3328, 27, "swiglu"),
    # fewer than 8 rows in a group on the K-stationary paths (the rows past B
    # repeat the last one and are never stored): whole K with 12 wavefronts,
    # two of them past the last step; whole K with 16; K ranges + reduce
    ("q4", 6144, 2560, 5, "rms"), ("q4", 2560, 4096, 3, "plain"), ("q4", 21504, 5376, 5, "plain"),
    ("q4", 19456, 2560, 7, "swiglu"),
    # activation rows with a stride past K (ld_x = K + 64) on each kernel
    ("q4", 6144, 2560, 8, "rms_strided"), ("q4", 21504, 5376, 8, "plain_strided"),
    ("q4", 2560, 4096, 8, "plain_strided"), ("q4", 2560, 9728, 8, "rms_strided"),
    ("q8", 1000, 2560, 8, "plain_strided"), ("q4", 4100, 1024, 20, "rms_strided"),
]


def _fused_inputs(fmt, n, k, b, op, seed):
    gen = synth.q4_0_matrix if fmt == "q4" else synth.q8_0_matrix
    W = gen(seed, f"t.batched.{fmt}.{n}.{k}", n, k)
    ld = 2 * k if op in ("swiglu", "geglu") else k + 64 if op.endswith("_strided") else k
    xa = synth.normal_f32(seed, f"t.batched.x.{k}.{b}", (b, ld)) * 2.0
    w = synth.uniform_f32(seed, f"t.batched.w.{k}", (k,), 0.8, 1.2)
    r = synth.normal_f32(seed, f"t.batched.r.{n}.{b}", (b, n))
    if op == "swiglu":
        xin = np.stack([oracle.swiglu(xa[i, :k], xa[i, k:]) for i in range(b)])
    elif op == "geglu":
        xin = np.stack([oracle.geglu(xa[i, :k], xa[i, k:]) for i in range(b)])
    elif op in ("plain", "plain_strided"):
        xin = xa[:, :k].astype(np.float64)
    else:
        xin = oracle.rmsnorm(xa[:, :k], None if op == "rms_unit" else w, 1e-6)
    return W, xa, w, r, xin, ld


_KIND = {"plain": q.IN_PLAIN, "rms": q.IN_RMSNORM, "rms_unit": q.IN_RMSNORM, "swiglu": q.IN_SWIGLU,
         "geglu": q.IN_GEGLU, "plain_strided": q.IN_PLAIN, "rms_strided": q.IN_RMSNORM}


@pytest.mark.parametrize("fmt,n,k,b,op", BATCHED_CASES)
def test_matvec_batched_parity(dev, fmt, n, k, b, op):
    _say(f"{fmt} batched {op} N={n} K={k} B={b}")
    orc = oracle.q4_0_matvec if fmt == "q4" else oracle.q8_0_matvec
    fn = q.q4_0_matvec_batched if fmt == "q4" else q.q8_0_matvec_batched
    W, xa, w, r, xin, ld = _fused_inputs(fmt, n, k, b, op, 107)
    ref, terms = orc(W, n, k, xin, res=r)
    xd = torch.from_numpy(xa).to(dev)
    yr = torch.from_numpy(r).to(dev)
    Wd = torch.from_numpy(W).to(dev)
    kw = dict(x2=xd[:, k:] if op in ("swiglu", "geglu") else None,
              norm_w=torch.from_numpy(w).to(dev) if op in ("rms", "rms_strided") else None, eps=1e-6)
    y0 = fn(Wd, xd, k, b, ld, _KIND[op], **kw)
    fn(Wd, xd, k, b, ld, _KIND[op], y=yr, residual=yr, **kw)
    torch.cuda.synchronize()
    _check(yr, ref, terms, f"{fmt} batched {op} {n}x{k} B={b}")
    # without the residual, and bitwise repeatable
    y1 = fn(Wd, xd, k, b, ld, _KIND[op], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "repeated launches differ bitwise"
    ref0, terms0 = orc(W, n, k, xin)
    _check(y0, ref0, terms0, f"{fmt} batched {op} {n}x{k} B={b} no residual")


def test_matvec_batched_row_scales(dev):
    """Rows of very different magnitude (and an all-zero row) keep the
    relative accuracy: each row is scaled by its own power of two."""
    _say("q4 batched row scales")
    n, k, b = 200, 2048, 6
    W = synth.q4_0_matrix(108, "t.batched.scales", n, k)
    x = synth.normal_f32(108, "t.batched.scales.x", (b, k))
    x = x * np.array([1.0, 3e4, 1e-6, 0.0, 7e-3, 1e9], dtype=np.float32)[:, None]
    ref, terms = oracle.q4_0_matvec(W, n, k, x)
    y = q.q4_0_matvec_batched(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev), k, b, k)
    torch.cuda.synchronize()
    _check(y, ref, terms, "row scales")
    assert torch.all(y[3] == 0)


def test_matvec_batched_matches_fused_path(dev):
    """The matrix-core path and the vector path agree within the bound on the
    attention-output shape of the 4B model at B = 8."""
    _say("batched vs fused, 2560x4096 B=8")
    n, k, b = 2560, 4096, 8
    W = torch.from_numpy(synth.q4_0_matrix(109, "t.batched.vs", n, k)).to(dev)
    x = torch.from_numpy(synth.normal_f32(109, "t.batched.vs.x", (b, k))).to(dev)
    y1 = q.q4_0_matvec_batched(W, x, k, b, k)
    y2 = q.q4_0_matvec(W, x)
    torch.cuda.synchronize()
    ref, terms = oracle.q4_0_matvec(W.cpu().numpy(), n, k, x.cpu().numpy())
    _check(y1, ref, terms, "batched")
    _check(y2, ref, terms, "fused")


@pytest.mark.parametrize("b", [8, 16, 32])
def test_matvec_batched_5376x21504_full(dev, b):
    """The 31B FFN-shape workload at B = 8 (the bench's B = 8 line) and at 16
    and 32 rows (batch groups), every output, bitwise repeatable."""
    _say(f"q4_0_matvec_batched 5376x21504 B={b} full")
    w = wl.MATVEC_5376x21504
    W, x = wl.matvec_inputs(w, b)
    ref, terms = oracle.q4_0_matvec(W, w.n, w.k, x)
    Wd = torch.from_numpy(W).to(dev)
    xd = torch.from_numpy(x).to(dev)
    y1 = q.q4_0_matvec_batched(Wd, xd, w.k, b, w.k)
    y2 = q.q4_0_matvec_batched(Wd, xd, w.k, b, w.k)
    torch.cuda.synchronize()
    _check(y1, ref, terms, f"5376x21504 B={b} batched")
    assert torch.equal(y1, y2)


def test_matvec_batched_workspace_errors(dev):
    n, k, b = 100, 512, 4
    W = torch.from_numpy(synth.q4_0_matrix(110, "t.batched.err", n, k)).to(dev)
    x = torch.zeros((b, k), dtype=torch.float32, device=dev)
    need = q.matvec_batched_workspace(n, k, b)
    small = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(q.Q4Error) as e:
        q.q4_0_matvec_batched(W, x, k, b, k, ws=small)
    assert e.value.status_name == "Q4_ERR_WORKSPACE"
    with pytest.raises(q.Q4Error) as e:
        q.q4_0_matvec_batched(torch.zeros((n, 9 * 18), dtype=torch.uint8, device=dev),
                              torch.zeros((b, 288), dtype=torch.float32, device=dev), 288, b, 288)
    assert e.value.status_name == "Q4_ERR_UNSUPPORTED"


def test_matvec_batched_spikes(dev):
    """One large element per 256-k step in a row of small ones: the step's
    power-of-two scale must come from the maximum over the whole step (every
    lane group and wavefront), or the spike overflows binary16."""
    _say("q4/q8 batched spikes")
    n, k, b = 130, 1024, 8
    x = synth.normal_f32(111, "t.batched.spike.x", (b, k)) * np.float32(1e-3)
    for r in range(b):
        for step in range(k // 256):
            x[r, step * 256 + (37 * r + 61 * step) % 256] = np.float32(3e4 * (1 + r))
    for fmt, gen, orc, fn in (("q4", synth.q4_0_matrix, oracle.q4_0_matvec, q.q4_0_matvec_batched),
                              ("q8", synth.q8_0_matrix, oracle.q8_0_matvec, q.q8_0_matvec_batched)):
        W = gen(111, f"t.batched.spike.{fmt}", n, k)
        ref, terms = orc(W, n, k, x)
        y = fn(torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev), k, b, k)
        torch.cuda.synchronize()
        _check(y, ref, terms, f"{fmt} spikes")


GLU_CASES = [
    # (path, N, K, B, op): merged gate|up with the SwiGLU output; N = 2F.
    # fused: the workspace-free q4_0_matvec_fused (the vector kernel, or from
    # B = 3 with many rows the matrix-core tile kernel over the whole K);
    # batched: q4_0_matvec_batched
    ("fused", 2 * 9728, 2560, 1, "rms"), ("fused", 2 * 300, 5376, 1, "rms"),
    ("fused", 2 * 77, 2048, 3, "plain"), ("fused", 2 * 33, 256, 8, "rms_unit"),
    ("fused", 2 * 8200, 2560, 4, "rms"), ("fused", 2 * 2050, 1024, 8, "plain"),
    ("batched", 2 * 9728, 2560, 8, "rms"), ("batched", 2 * 300, 2560, 8, "rms"),
    ("batched", 2 * 77, 9728, 5, "plain"), ("batched", 2 * 1000, 5376, 2, "rms"),
    ("batched", 2 * 33, 256, 1, "swiglu"),
    ("batched", 2 * 16384, 2048, 8, "rms"), ("batched", 2 * 16500, 1024, 4, "plain"),
    ("batched", 2 * 9728, 2560, 32, "rms"), ("batched", 2 * 300, 2560, 11, "plain"),
    # K-stationary kernel with K ranges added by the second launch
    ("batched", 2 * 8200, 5376, 8, "rms"), ("batched", 2 * 8210, 3328, 13, "plain"),
    ("batched", 2 * 8200, 3328, 32, "rms"), ("batched", 2 * 4100, 2048, 16, "plain"),
]


@pytest.mark.parametrize("path,n,k,b,op", GLU_CASES)
def test_matvec_swiglu_output(dev, path, n, k, b, op):
    """y[p] = SiLU(z[p]) * z[p + N/2] with z the matvec: bound from the two
    matvec bounds through SiLU(g) u (|SiLU'| <= 1.1) plus 2e-4 relative."""
    _say(f"{path} swiglu output {op} N={n} K={k} B={b}")
    W, xa, w, r, xin, ld = _fused_inputs("q4", n, k, b, op, 112)
    z, t = oracle.q4_0_matvec(W, n, k, xin)
    F = n // 2
    g, u = z[:, :F], z[:, F:]
    tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
    ref = g / (1.0 + np.exp(-g)) * u
    tol = 1.1 * tg * np.abs(u) + np.abs(g / (1.0 + np.exp(-g))) * tu + 2e-4 * np.abs(ref) + 1e-6
    xd = torch.from_numpy(xa).to(dev)
    fn = q.q4_0_matvec_batched if path == "batched" else q.q4_0_matvec_fused
    kw = dict(x2=xd[:, k:] if op in ("swiglu", "geglu") else None,
              norm_w=torch.from_numpy(w).to(dev) if op == "rms" else None, eps=1e-6)
    h = fn(torch.from_numpy(W).to(dev), xd, k, b, ld, _KIND[op], out_op=q.OUT_SWIGLU, **kw)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64)
    assert got.shape == (b, F)
    ratio = float((np.abs(got - ref) / tol).max())
    assert np.all(np.isfinite(got)) and ratio <= 1.0, f"max err/tol {ratio:.3e}"



GEGLU_OUT_CASES = [
    # (path, N, K, B, op): merged gate|up with the GeGLU output (tanh-form GELU gate)
    ("fused", 2 * 9728, 2560, 1, "rms"), ("fused", 2 * 77, 2048, 3, "plain"),
    ("fused", 2 * 8200, 2560, 5, "rms"),
    ("batched", 2 * 9728, 2560, 8, "rms"), ("batched", 2 * 1000, 5376, 2, "rms"),
    ("batched", 2 * 16384, 2048, 8, "rms"), ("batched", 2 * 300, 2560, 11, "plain"),
    ("batched", 2 * 8200, 5376, 3, "plain"), ("batched", 2 * 4100, 1024, 32, "rms"),
]


@pytest.mark.parametrize("path,n,k,b,op", GEGLU_OUT_CASES)
def test_matvec_geglu_output(dev, path, n, k, b, op):
    """y[p] = gelu(z[p]) * z[p + N/2]: bound from the two matvec bounds through
    gelu(g) u (|gelu'| <= 1.13 for the tanh form) plus 2e-4 relative."""
    _say(f"{path} geglu output {op} N={n} K={k} B={b}")
    W, xa, w, r, xin, ld = _fused_inputs("q4", n, k, b, op, 117)
    z, t = oracle.q4_0_matvec(W, n, k, xin)
    F = n // 2
    g, u = z[:, :F], z[:, F:]
    tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
    ref = oracle.geglu(g, u)
    gel = np.abs(oracle.geglu(g, np.ones_like(g)))
    tol = 1.13 * tg * np.abs(u) + gel * tu + 2e-4 * np.abs(ref) + 1e-6
    xd = torch.from_numpy(xa).to(dev)
    fn = q.q4_0_matvec_batched if path == "batched" else q.q4_0_matvec_fused
    kw = dict(norm_w=torch.from_numpy(w).to(dev) if op == "rms" else None, eps=1e-6)
    h = fn(torch.from_numpy(W).to(dev), xd, k, b, ld, _KIND[op], out_op=q.OUT_GEGLU, **kw)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64)
    assert got.shape == (b, F)
    ratio = float((np.abs(got - ref) / tol).max())
    assert np.all(np.isfinite(got)) and ratio <= 1.0, f"max err/tol {ratio:.3e}"


# (N, K, B, output transform, pre-norm gain): ragged rows, every JX (K = 256 .. 8192),
# B up to 8, gated outputs, a unit pre-norm gain
POST_NORM_CASES = [(300, 256, 1, "plain", True), (1027, 5376, 1, "plain", True),
                   (1026, 2048, 3, "swiglu", True), (1400, 1024, 2, "geglu", False),
                   (96, 8192, 1, "plain", True), (64, 768, 8, "plain", True)]


@pytest.mark.parametrize("n,k,b,out,gain", POST_NORM_CASES)
def test_matvec_post_norm(dev, n, k, b, out, gain):
    """h_out = h + pw * rmsnorm(z) against the oracle's post-norm add; y against the
    oracle's matvec of pre_w * rmsnorm(h_out) fed the GPU's h_out (bounds as for the
    fused RMSNorm matvec and the gated outputs); h_out's row padding is not written."""
    _say(f"post-norm matvec {out} N={n} K={k} B={b}")
    W = synth.q4_0_matrix(121, f"pn.W.{n}.{k}", n, k)
    ld = k + 32
    h = synth.normal_f32(121, f"pn.h.{k}.{b}", (b, ld))
    z = synth.normal_f32(121, f"pn.z.{k}.{b}", (b, ld)) * 3.0
    pw = synth.uniform_f32(121, f"pn.pw.{k}", (k,), 0.8, 1.2)
    gw = synth.uniform_f32(121, f"pn.gw.{k}", (k,), 0.8, 1.2) if gain else None
    hod = torch.zeros((b, ld), dtype=torch.float32, device=dev)
    oo = {"plain": q.OUT_PLAIN, "swiglu": q.OUT_SWIGLU, "geglu": q.OUT_GEGLU}[out]
    y = q.q4_0_matvec_post_norm(torch.from_numpy(W).to(dev), torch.from_numpy(h).to(dev),
                                torch.from_numpy(z).to(dev), k, b, ld, torch.from_numpy(pw).to(dev),
                                torch.from_numpy(gw).to(dev) if gain else None, 1e-6, hod,
                                out_op=oo)
    torch.cuda.synchronize()
    ho = hod.cpu().numpy().astype(np.float64)
    assert np.all(ho[:, k:] == 0.0)
    normed = oracle.rmsnorm(z[:, :k], pw, 1e-6)
    ref_h = h[:, :k].astype(np.float64) + normed
    assert np.all(np.abs(ho[:, :k] - ref_h) <= 2e-4 * np.abs(normed) + 2.0 ** -23 * np.abs(ref_h) + 1e-6)
    zz, t = oracle.q4_0_matvec(W, n, k, oracle.rmsnorm(ho[:, :k], gw, 1e-6))
    got = y.cpu().numpy().astype(np.float64)
    if out == "plain":
        ref, tol = zz, 2e-4 * t + 1e-6
    else:
        F = n // 2
        g, u = zz[:, :F], zz[:, F:]
        tg, tu = 2e-4 * t[:, :F] + 1e-6, 2e-4 * t[:, F:] + 1e-6
        act = oracle.swiglu if out == "swiglu" else oracle.geglu
        ref = act(g, u)
        tol = 1.13 * tg * np.abs(u) + np.abs(act(g, np.ones_like(g))) * tu + 2e-4 * np.abs(ref) + 1e-6
    assert got.shape == ref.shape
    ratio = float((np.abs(got - ref) / tol).max())
    assert np.all(np.isfinite(got)) and ratio <= 1.0, f"max err/tol {ratio:.3e}"


def test_q8_0_gather_scaled(dev):
    """Rows times a scale (the Gemma-4 sqrt(d) embedding scale): (d q) s in fp32,
    within one rounding of the exact product."""
    _say("q8_0_gather_scaled")
    v, k = 1000, 5376
    E = synth.q8_0_matrix(108, "t.gather_s", v, k)
    tok = np.array([0, 999, 17, 512], dtype=np.int32)
    s = float(np.float32(np.sqrt(5376.0)))
    ref = oracle.q8_0_gather(E, v, k, tok) * s
    x = q.q8_0_gather(torch.from_numpy(E).to(dev), torch.from_numpy(tok).to(dev), k, scale=s)
    torch.cuda.synchronize()
    got = x.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -24 * np.abs(ref))
