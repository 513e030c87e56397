"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

import q4_quantized_matvec_amd as q
from q4_quantized_matvec_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "q4dec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_parsed():
    names = declared_functions()
    for must in ("q4_0_matvec", "q8_0_matvec", "rmsnorm", "qk_norm_rope", "gqa_decode_attn",
                 "swiglu", "decode_step", "argmax_rows", "q8_0_gather"):
        assert must in names


def test_exports_every_declared_symbol():
    cdll = C.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(cdll, n)]
    assert not missing, f"not exported: {missing}"
    assert set(declared_functions()) <= set(_lib._SIGS)


def test_version_string():
    assert "gfx950" in q.version()


def _status(fn, *args):
    st = fn(*args)
    return _lib.STATUS[st], q.lib().q4dec_last_error().decode()


def test_matvec_rejects_bad_arguments_on_host():
    L = q.lib()
    fake = 0x1000  # never dereferenced: validation fails first
    assert _status(L.q4_0_matvec, None, 4, 32, fake, 1, fake, None, None)[0] == "Q4_ERR_INVALID_ARG"
    assert _status(L.q4_0_matvec, fake, 0, 32, fake, 1, fake, None, None)[0] == "Q4_ERR_INVALID_ARG"
    assert _status(L.q4_0_matvec, fake, 4, 48, fake, 1, fake, None, None)[0] == "Q4_ERR_SHAPE"
    assert _status(L.q4_0_matvec, fake, 4, 32, fake, 9, fake, None, None)[0] == "Q4_ERR_UNSUPPORTED"
    assert _status(L.q4_0_matvec, fake + 1, 4, 32, fake, 1, fake, None, None)[0] == "Q4_ERR_ALIGNMENT"
    st, msg = _status(L.q8_0_matvec, fake, 4, 32, fake + 2, 1, fake, None, None)
    assert st == "Q4_ERR_ALIGNMENT" and "aligned" in msg
    assert _status(L.q8_0_gather, fake, 10, 33, fake, 1, fake, None)[0] == "Q4_ERR_SHAPE"
    assert _status(L.q8_0_gather, None, 10, 32, fake, 1, fake, None)[0] == "Q4_ERR_INVALID_ARG"


def test_batched_matvec_rejects_bad_arguments_on_host():
    L = q.lib()
    fake = 0x10000
    need = q.matvec_batched_workspace(100, 512, 4)
    assert need > 0
    assert q.matvec_batched_workspace(100, 288, 4) == 0    # K % 256 != 0
    assert q.matvec_batched_workspace(100, 512, 33) == 0   # B > 32
    assert q.matvec_batched_workspace(100, 512, 32) > 0
    ybuf = 0x40000000  # does not overlap x
    args = lambda W, K, B, ws, nbytes: (W, 100, K, fake, None, K, B, 0, 0, None, 0.0, ybuf, None,
                                        ws, nbytes, None)
    assert _status(L.q4_0_matvec_batched, *args(fake, 512, 4, fake, need - 1))[0] == "Q4_ERR_WORKSPACE"
    assert _status(L.q4_0_matvec_batched, *args(fake, 512, 4, fake + 16, need))[0] == "Q4_ERR_WORKSPACE"
    assert _status(L.q4_0_matvec_batched, *args(fake, 288, 4, fake, need))[0] == "Q4_ERR_UNSUPPORTED"
    assert _status(L.q4_0_matvec_batched, *args(fake, 512, 33, fake, need))[0] == "Q4_ERR_UNSUPPORTED"
    assert _status(L.q8_0_matvec_batched, *args(fake + 2, 512, 4, fake, need))[0] == "Q4_ERR_ALIGNMENT"
    assert _status(L.q4_0_matvec_batched, *args(None, 512, 4, fake, need))[0] == "Q4_ERR_INVALID_ARG"


def test_swiglu_output_rejected_where_unsupported():
    L = q.lib()
    fake, ybuf = 0x10000, 0x40000000
    fused = lambda N, K, res: (fake, N, K, fake, None, K, 1, 0, 1, None, 0.0, ybuf, res, None)
    assert _status(L.q4_0_matvec_fused, *fused(101, 512, None))[0] == "Q4_ERR_INVALID_ARG"   # odd N
    assert _status(L.q4_0_matvec_fused, *fused(100, 512, ybuf))[0] == "Q4_ERR_INVALID_ARG"  # residual
    assert _status(L.q4_0_matvec_fused, *fused(100, 16384, None))[0] == "Q4_ERR_UNSUPPORTED"
    assert _status(L.q4_0_matvec_fused, fake, 100, 512, fake, None, 512, 1, 0, 3, None, 0.0, ybuf,
                   None, None)[0] == "Q4_ERR_INVALID_ARG"                                     # bad out_op
    assert _status(L.q4_0_matvec_fused, fake, 101, 512, fake, None, 512, 1, 0, 2, None, 0.0, ybuf,
                   None, None)[0] == "Q4_ERR_INVALID_ARG"                                     # GeGLU, odd N
    assert _status(L.q4_0_matvec_fused, fake, 100, 512, fake, None, 512, 1, 4, 0, None, 0.0, ybuf,
                   None, None)[0] == "Q4_ERR_INVALID_ARG"                                     # bad op
    assert _status(L.q4_0_matvec_fused, fake, 100, 512, fake, None, 512, 1, 3, 0, None, 0.0, ybuf,
                   None, None)[0] == "Q4_ERR_INVALID_ARG"                                     # GeGLU, no x2


def test_post_norm_matvec_rejects_bad_arguments_on_host():
    """q4_0_matvec_post_norm: NULLs, K limits of the staged row, B > 8, odd N with a gated
    output, alignment, and h_out overlapping h or z (other workgroups read them)."""
    L = q.lib()
    W, h, z, ho, pw, y = 0x10000, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000

    def st(W=W, N=64, K=512, h=h, z=z, ld=512, B=1, pw=pw, ho=ho, out=0, y=y):
        return _status(L.q4_0_matvec_post_norm, W, N, K, h, z, ld, B, pw, None, 1e-6, ho, out, y,
                       None)[0]
    assert st(h=None) == "Q4_ERR_INVALID_ARG"
    assert st(pw=None) == "Q4_ERR_INVALID_ARG"
    assert st(ho=None) == "Q4_ERR_INVALID_ARG"
    assert st(K=288, ld=288) == "Q4_ERR_UNSUPPORTED"      # K % 256
    assert st(K=8448, ld=8448) == "Q4_ERR_UNSUPPORTED"    # K > 8192
    assert st(B=9) == "Q4_ERR_UNSUPPORTED"
    assert st(N=65, out=1) == "Q4_ERR_INVALID_ARG"        # gated output, odd N
    assert st(out=3) == "Q4_ERR_INVALID_ARG"
    assert st(ld=256) == "Q4_ERR_SHAPE"
    assert st(h=h + 4) == "Q4_ERR_ALIGNMENT"
    assert st(ld=514) == "Q4_ERR_ALIGNMENT"
    assert st(ho=h + 1024) == "Q4_ERR_INVALID_ARG"        # h_out inside h's rows
    assert st(ho=z) == "Q4_ERR_INVALID_ARG"
    assert st(y=ho + 16) == "Q4_ERR_INVALID_ARG"


def test_gemma_variant_ops_reject_bad_arguments_on_host():
    import ctypes as C
    L = q.lib()
    a, b = 0x10000, 0x20000
    assert _status(L.rmsnorm_add, a, None, 4, 100, 1e-6, a + 200, None)[0] == "Q4_ERR_INVALID_ARG"  # overlap
    assert _status(L.rmsnorm_add, a, None, 4, 100, -1.0, b, None)[0] == "Q4_ERR_INVALID_ARG"      # eps
    assert _status(L.softcap, a, 10, 0.0, None)[0] == "Q4_ERR_INVALID_ARG"                       # cap
    assert _status(L.softcap, a + 2, 10, 30.0, None)[0] == "Q4_ERR_ALIGNMENT"
    assert _status(L.geglu, a, None, 1, 8, 8, b, None)[0] == "Q4_ERR_INVALID_ARG"
    kv = _lib.KVLayout(1, 2, 128, 16, 4096, 2048, 128, 0)
    args = lambda rot: (a, 512, a, a, 512, a, a, 4, C.byref(kv), b, 1e4, 1e-6, 0, rot, a, a, None)
    for rot in (0, 3, 130):  # too small, odd, beyond head_dim
        assert _status(L.qk_norm_rope_partial, *args(rot))[0] == "Q4_ERR_INVALID_ARG"


def test_decode_model_batch_limits_on_host():
    """Up to 8 sequences any shape; up to 32 only where every projection runs
    on the matrix cores (K multiples of 256, 16-byte aligned weights)."""
    import ctypes as C
    L = q.lib()
    fake = 0x100000  # never dereferenced: sizes only

    def status(batch, d_model=256, ffn=512, hd=64, wq_off=0):
        ly = (_lib.LayerDesc * 1)()
        l0 = ly[0]
        for f in ("wqkv", "wo", "wgu", "wd", "attn_norm", "ffn_norm", "q_norm", "k_norm",
                  "k_cache", "v_cache"):
            setattr(l0, f, fake)
        l0.wqkv = fake + wq_off
        l0.n_kv_heads, l0.head_dim, l0.cap, l0.window = 2, hd, 64, 0
        l0.rope_theta, l0.attn_scale, l0.v_from_k = 1e4, 0.125, 0
        d = _lib.ModelDesc(1, d_model, 4, ffn, 1000, batch, 1e-6, fake, fake,
                           C.cast(ly, C.POINTER(_lib.LayerDesc)))
        nbytes = C.c_size_t()
        return _status(L.decode_model_workspace, C.byref(d), C.byref(nbytes))[0]

    assert status(8) == "Q4_OK" and status(16) == "Q4_OK" and status(32) == "Q4_OK"
    assert status(33) == "Q4_ERR_UNSUPPORTED"
    assert status(8, d_model=288) == "Q4_OK"
    assert status(9, d_model=288) == "Q4_ERR_UNSUPPORTED"      # d_model % 256
    assert status(16, ffn=544) == "Q4_ERR_UNSUPPORTED"         # ffn % 256
    assert status(16, hd=64, d_model=256, wq_off=2) == "Q4_ERR_UNSUPPORTED"  # 2-byte aligned wqkv
    assert status(8, wq_off=2) == "Q4_OK"


def test_decode_model_variant_options_on_host():
    import ctypes as C
    L = q.lib()
    fake = 0x100000

    def status(ffn_act=0, embed_scale=0.0, softcap=0.0, rope_dims=0, post=0):
        ly = (_lib.LayerDesc * 1)()
        l0 = ly[0]
        for f in ("wqkv", "wo", "wgu", "wd", "attn_norm", "ffn_norm", "q_norm", "k_norm",
                  "k_cache", "v_cache"):
            setattr(l0, f, fake)
        l0.n_kv_heads, l0.head_dim, l0.cap, l0.window = 2, 64, 64, 0
        l0.rope_theta, l0.attn_scale, l0.v_from_k, l0.rope_dims = 1e4, 0.125, 0, rope_dims
        l0.post_attn_norm = fake + post if post else None
        d = _lib.ModelDesc(1, 256, 4, 512, 1000, 2, 1e-6, fake, fake,
                           C.cast(ly, C.POINTER(_lib.LayerDesc)), ffn_act, embed_scale, softcap)
        nbytes = C.c_size_t()
        return _status(L.decode_model_workspace, C.byref(d), C.byref(nbytes))[0]

    assert status() == "Q4_OK"
    assert status(ffn_act=1, embed_scale=16.0, softcap=30.0, rope_dims=16, post=0x100) == "Q4_OK"
    assert status(ffn_act=2) == "Q4_ERR_INVALID_ARG"
    assert status(softcap=-1.0) == "Q4_ERR_INVALID_ARG"
    assert status(rope_dims=15) == "Q4_ERR_INVALID_ARG"
    assert status(rope_dims=66) == "Q4_ERR_INVALID_ARG"
    assert status(post=2) == "Q4_ERR_ALIGNMENT"


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu_visible(), reason="needs a machine without a GPU")
def test_hip_runtime_error_is_reported_as_q4_err_hip():
    """Valid, aligned arguments pass host validation and reach the HIP
    runtime, which has no device here: the call returns Q4_ERR_HIP with the
    runtime's message instead of crashing.  The buffers are host memory that
    no kernel ever touches (the launch itself fails)."""
    import numpy as np
    L = q.lib()
    W = np.zeros(64 * 8 * 18, np.uint8)
    x = np.zeros((2, 256), np.float32)
    y = np.zeros((2, 64), np.float32)
    st, msg = _status(L.q4_0_matvec, W.ctypes.data, 64, 256, x.ctypes.data, 1, y.ctypes.data,
                      None, None)
    assert st == "Q4_ERR_HIP" and "device" in msg.lower()
    st, msg = _status(L.q4_0_matvec_batched_noalloc, W.ctypes.data, 64, 256, x.ctypes.data, None,
                      256, 2, 0, 0, None, 0.0, y.ctypes.data, None, None)
    assert st == "Q4_ERR_HIP" and msg
