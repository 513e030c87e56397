"""The allocation-free batched matvec (static per-device scratch) against the
workspace entry point it varies: bit-identical outputs on two calls in a row,
the second with a smaller input, and the oracle's bound on the first."""
import numpy as np
import pytest
import torch

import oracle
import q4_quantized_matvec_amd as q
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(dev, seed, N, K, B, op, residual):
    W = synth.q4_0_matrix(seed, "noalloc.W", N, K)
    x = synth.normal_f32(seed, "noalloc.x", (B, K))
    g = synth.uniform_f32(seed, "noalloc.g", (K,), 0.8, 1.2)
    r = synth.normal_f32(seed, "noalloc.r", (B, N))
    Wd, xd, gd = (torch.from_numpy(a).to(dev) for a in (W, x, g))
    rd = torch.from_numpy(r).to(dev) if residual else None
    kw = dict(norm_w=gd if op == q.IN_RMSNORM else None, eps=1e-6, residual=rd)
    return W, x, g, r, Wd, xd, kw


def test_noalloc_matches_workspace_entry_point(dev):
    cases = [(20261210, 21504, 5376, 8, q.IN_RMSNORM, False),  # tile kernel, K split 6 ways
             (20261211, 1000, 2560, 3, q.IN_PLAIN, True)]       # smaller: shared-step kernel
    for i, (seed, N, K, B, op, residual) in enumerate(cases):
        _say(f"noalloc call {i}: N={N} K={K} B={B} op={op} residual={residual}")
        assert q.matvec_batched_workspace(N, K, B) <= q._lib.NOALLOC_SCRATCH_BYTES
        W, x, g, r, Wd, xd, kw = _case(dev, seed, N, K, B, op, residual)
        y0 = torch.full((B, N), float("nan"), device=dev)
        y1 = torch.full((B, N), float("nan"), device=dev)
        q.q4_0_matvec_batched_noalloc(Wd, xd, K, B, K, op, y=y0, **kw)
        q.q4_0_matvec_batched(Wd, xd, K, B, K, op, y=y1, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"call {i}: outputs differ"
        xin = oracle.rmsnorm(x.astype(np.float64), g, 1e-6) if op == q.IN_RMSNORM else x
        ref, terms = oracle.q4_0_matvec(W, N, K, xin, res=r if residual else None)
        ratio = float((np.abs(y0.cpu().numpy() - ref) / (2e-4 * terms + 1e-6)).max())
        _say(f"  bit-identical to q4_0_matvec_batched; max err/tol vs oracle {ratio:.3e}")
        assert ratio <= 1.0


def test_noalloc_rejects_shape_beyond_scratch(dev):
    N, K, B = 21504, 5376, 32
    need = q.matvec_batched_workspace(N, K, B)
    assert need > q._lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, K), device=dev)
    W = torch.zeros(N * K // 32 * 18, dtype=torch.uint8, device=dev)
    with pytest.raises(q.Q4Error) as e:
        q.q4_0_matvec_batched_noalloc(W, x, K, B, K, n=N)
    assert e.value.status_name == "Q4_ERR_UNSUPPORTED" and "scratch" in str(e.value)
