"""fp64 CPU oracle for the Q4_0 decode hot path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library (``q4_quantized_matvec_amd``)
never does and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain scalar C99, fp64); this module only
builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_dbl_p = C.POINTER(C.c_double)
_u8_p = C.POINTER(C.c_uint8)
_i32_p = C.POINTER(C.c_int32)
_f32_p = C.POINTER(C.c_float)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP over independent outputs)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Layer(C.Structure):
    _fields_ = [("wqkv", _u8_p), ("wo", _u8_p), ("wgu", _u8_p), ("wd", _u8_p),
                ("attn_norm", _dbl_p), ("ffn_norm", _dbl_p), ("q_norm", _dbl_p),
                ("k_norm", _dbl_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("n_kv_heads", C.c_int64), ("head_dim", C.c_int64), ("cap", C.c_int64),
                ("window", C.c_int64), ("rope_theta", C.c_double), ("attn_scale", C.c_double),
                ("v_from_k", C.c_int32), ("kv_f16", C.c_int32), ("rope_dims", C.c_int64),
                ("post_attn_norm", _dbl_p), ("post_ffn_norm", _dbl_p)]


class _Model(C.Structure):
    _fields_ = [("n_layers", C.c_int64), ("d_model", C.c_int64), ("n_q_heads", C.c_int64),
                ("ffn", C.c_int64), ("vocab", C.c_int64), ("batch", C.c_int64),
                ("eps", C.c_double), ("embed", _u8_p), ("final_norm", _dbl_p),
                ("layers", C.POINTER(_Layer)), ("ffn_act", C.c_int32),
                ("embed_scale", C.c_double), ("logit_softcap", C.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        L.orc_half_to_double.argtypes = [C.c_uint16]
        L.orc_half_to_double.restype = C.c_double
        L.orc_double_to_half.argtypes = [C.c_double]
        L.orc_double_to_half.restype = C.c_uint16
        for name in ("orc_q4_0_dequant", "orc_q8_0_dequant"):
            getattr(L, name).argtypes = [_u8_p, C.c_int64, C.c_int64, _dbl_p]
        for name in ("orc_q4_0_matvec", "orc_q8_0_matvec"):
            getattr(L, name).argtypes = [_u8_p, C.c_int64, C.c_int64, _dbl_p, C.c_int64,
                                         _dbl_p, _dbl_p, _dbl_p]
        L.orc_q8_0_gather.argtypes = [_u8_p, C.c_int64, C.c_int64, _i32_p, C.c_int64, _dbl_p]
        L.orc_rmsnorm.argtypes = [_dbl_p, _dbl_p, C.c_int64, C.c_int64, C.c_double, _dbl_p]
        L.orc_rope_neox.argtypes = [_dbl_p, C.c_int64, C.c_int64, C.c_double]
        L.orc_swiglu.argtypes = [_dbl_p, _dbl_p, C.c_int64, _dbl_p]
        L.orc_geglu.argtypes = [_dbl_p, _dbl_p, C.c_int64, _dbl_p]
        L.orc_softcap.argtypes = [_dbl_p, C.c_int64, C.c_double]
        L.orc_argmax.argtypes = [_dbl_p, C.c_int64, _dbl_p]
        L.orc_argmax.restype = C.c_int64
        L.orc_gqa_attention.argtypes = [_dbl_p, C.c_int64, C.c_int64, C.c_int64, _dbl_p,
                                        _dbl_p, C.c_int64, C.c_int64, C.c_double, _dbl_p,
                                        _dbl_p]
        L.orc_decode_step.argtypes = [C.POINTER(_Model), C.c_int64, _i32_p, _i32_p, _dbl_p,
                                      _dbl_p]
        L.orc_num_threads.restype = C.c_int
        L.orc_set_num_threads.argtypes = [C.c_int]
        L.orc_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later calls from this thread (results do not
    depend on it)."""
    lib().orc_set_num_threads(int(n))


def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(bits)


def double_to_half(v: float) -> int:
    """Bits of the binary16 nearest to v (ties to even)."""
    return lib().orc_double_to_half(float(v))


def q4_0_dequant(w, n_rows, k):
    w = _u8(w)
    assert w.size == n_rows * (k // 32) * 18
    out = np.empty((n_rows, k))
    lib().orc_q4_0_dequant(_p(w, _u8_p), n_rows, k, _p(out, _dbl_p))
    return out


def q8_0_dequant(w, n_rows, k):
    w = _u8(w)
    assert w.size == n_rows * (k // 32) * 34
    out = np.empty((n_rows, k))
    lib().orc_q8_0_dequant(_p(w, _u8_p), n_rows, k, _p(out, _dbl_p))
    return out


def _matvec(fn, bpb, w, n_rows, k, x, res):
    w = _u8(w)
    assert w.size == n_rows * (k // 32) * bpb
    x = _f64(x)
    if x.ndim == 1:
        x = x[None, :]
    batch = x.shape[0]
    assert x.shape[1] == k
    res = None if res is None else _f64(res).reshape(batch, n_rows)
    y = np.empty((batch, n_rows))
    terms = np.empty((batch, n_rows))
    fn(_p(w, _u8_p), n_rows, k, _p(x, _dbl_p), batch, _p(res, _dbl_p), _p(y, _dbl_p),
       _p(terms, _dbl_p))
    return y, terms


def q4_0_matvec(w, n_rows, k, x, res=None):
    """Returns (y[B,N], sum|w x|[B,N]) in fp64."""
    return _matvec(lib().orc_q4_0_matvec, 18, w, n_rows, k, x, res)


def q8_0_matvec(w, n_rows, k, x, res=None):
    return _matvec(lib().orc_q8_0_matvec, 34, w, n_rows, k, x, res)


def q8_0_gather(table, vocab, k, tok):
    table = _u8(table)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    out = np.empty((tok.size, k))
    lib().orc_q8_0_gather(_p(table, _u8_p), vocab, k, _p(tok, _i32_p), tok.size, _p(out, _dbl_p))
    return out


def rmsnorm(x, w, eps):
    x = _f64(x)
    dim = x.shape[-1]
    rows = x.size // dim
    w = None if w is None else _f64(w)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x, _dbl_p), _p(w, _dbl_p), rows, dim, eps, _p(y, _dbl_p))
    return y


def rope_neox(x, pos, theta, rot_dims=0):
    """Rotate every head vector (last axis) of x at position pos; with
    rot_dims (p-RoPE) only the first rot_dims elements rotate."""
    y = _f64(x).copy()
    hd = y.shape[-1]
    rot = rot_dims if rot_dims else hd
    flat = y.reshape(-1, hd)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib().orc_rope_neox(_p(row, _dbl_p), rot, int(pos), theta)
        flat[r] = row
    return flat.reshape(y.shape)


def swiglu(g, u):
    g = _f64(g)
    u = _f64(u)
    h = np.empty_like(g)
    lib().orc_swiglu(_p(g, _dbl_p), _p(u, _dbl_p), g.size, _p(h, _dbl_p))
    return h


def geglu(g, u):
    g = _f64(g)
    u = _f64(u)
    h = np.empty_like(g)
    lib().orc_geglu(_p(g, _dbl_p), _p(u, _dbl_p), g.size, _p(h, _dbl_p))
    return h


def softcap(v, c):
    y = _f64(v).copy()
    lib().orc_softcap(_p(y, _dbl_p), y.size, float(c))
    return y


def argmax(v):
    v = _f64(v)
    m = C.c_double()
    i = lib().orc_argmax(_p(v, _dbl_p), v.size, C.byref(m))
    return int(i), m.value


def gqa_attention(q, keys, values, window, scale):
    """q [Hq, hd]; keys/values [n_pos, Hkv, hd] (position-indexed).

    Returns (o [Hq, hd], bound [Hq, hd]).
    """
    q = _f64(q)
    keys = _f64(keys)
    values = _f64(values)
    hq, hd = q.shape
    n_pos, hkv, hd2 = keys.shape
    assert hd2 == hd and values.shape == keys.shape and n_pos >= 1
    o = np.empty((hq, hd))
    bound = np.empty((hq, hd))
    lib().orc_gqa_attention(_p(q, _dbl_p), hq, hkv, hd, _p(keys, _dbl_p), _p(values, _dbl_p),
                            n_pos, int(window), float(scale), _p(o, _dbl_p), _p(bound, _dbl_p))
    return o, bound


class Model:
    """Owns the ctypes view of a decode model for orc_decode_step.

    ``spec``: dict with d_model, n_q_heads, ffn, vocab, batch, eps, embed (uint8),
    final_norm, layers (list of dicts with wqkv, wo, wgu, wd, attn_norm, ffn_norm,
    q_norm, k_norm, k_cache, v_cache (float32 or float16 [B, Hkv, cap, hd], modified in
    place), n_kv_heads, head_dim, window, rope_theta, attn_scale, v_from_k).
    """

    def __init__(self, spec):
        self._keep = []
        layers = (_Layer * len(spec["layers"]))()
        for i, L in enumerate(spec["layers"]):
            arrs = {}
            for key in ("wqkv", "wo", "wgu", "wd"):
                arrs[key] = _u8(L[key])
            for key in ("attn_norm", "ffn_norm", "q_norm", "k_norm"):
                arrs[key] = _f64(L[key])
            kc, vc = L["k_cache"], L["v_cache"]
            assert kc.dtype in (np.float32, np.float16) and kc.flags.c_contiguous
            assert vc.dtype == kc.dtype and vc.flags.c_contiguous
            self._keep.append(arrs)
            ly = layers[i]
            for key in ("wqkv", "wo", "wgu", "wd"):
                setattr(ly, key, _p(arrs[key], _u8_p))
            for key in ("attn_norm", "ffn_norm", "q_norm", "k_norm"):
                setattr(ly, key, _p(arrs[key], _dbl_p))
            ly.k_cache = kc.ctypes.data
            ly.v_cache = vc.ctypes.data
            ly.kv_f16 = 1 if kc.dtype == np.float16 else 0
            ly.n_kv_heads = L["n_kv_heads"]
            ly.head_dim = L["head_dim"]
            ly.cap = kc.shape[2]
            ly.window = L["window"]
            ly.rope_theta = L["rope_theta"]
            ly.attn_scale = L["attn_scale"]
            ly.v_from_k = 1 if L["v_from_k"] else 0
            # Gemma-4 block variants (absent keys: the plain pre-norm block)
            ly.rope_dims = int(L.get("rope_dims", 0) or 0)
            for key in ("post_attn_norm", "post_ffn_norm"):
                if L.get(key) is not None:
                    arrs[key] = _f64(L[key])
                    setattr(ly, key, _p(arrs[key], _dbl_p))
        self._layers = layers
        self.embed = _u8(spec["embed"])
        self.final_norm = _f64(spec["final_norm"])
        m = _Model()
        m.n_layers = len(spec["layers"])
        m.d_model = spec["d_model"]
        m.n_q_heads = spec["n_q_heads"]
        m.ffn = spec["ffn"]
        m.vocab = spec["vocab"]
        m.batch = spec["batch"]
        m.eps = spec["eps"]
        m.embed = _p(self.embed, _u8_p)
        m.final_norm = _p(self.final_norm, _dbl_p)
        m.layers = C.cast(layers, C.POINTER(_Layer))
        m.ffn_act = {"silu": 0, "gelu_tanh": 1}[spec.get("ffn_act", "silu")]
        m.embed_scale = float(spec.get("embed_scale", 0.0) or 0.0)
        m.logit_softcap = float(spec.get("logit_softcap", 0.0) or 0.0)
        self._m = m
        self.batch = spec["batch"]
        self.vocab = spec["vocab"]

    def step(self, pos, tok, want_logits=False):
        tok = np.ascontiguousarray(tok, dtype=np.int32)
        nxt = np.empty(self.batch, dtype=np.int32)
        margins = np.empty(self.batch)
        logits = np.empty((self.batch, self.vocab)) if want_logits else None
        lib().orc_decode_step(C.byref(self._m), int(pos), _p(tok, _i32_p), _p(nxt, _i32_p),
                              _p(logits, _dbl_p), _p(margins, _dbl_p))
        return nxt, logits, margins
