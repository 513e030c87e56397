"""ctypes view of libq4dec.so.  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4dec.so")

STATUS = {
    0: "Q4_OK", 1: "Q4_ERR_INVALID_ARG", 2: "Q4_ERR_SHAPE", 3: "Q4_ERR_ALIGNMENT",
    4: "Q4_ERR_CAPACITY", 5: "Q4_ERR_WORKSPACE", 6: "Q4_ERR_UNSUPPORTED", 7: "Q4_ERR_HIP",
}


class Q4Error(RuntimeError):
    def __init__(self, name, status, msg):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{name}: {self.status_name}: {msg}")


KV_F32, KV_F16 = 0, 1


class KVLayout(C.Structure):
    _fields_ = [("batch", C.c_int64), ("n_kv_heads", C.c_int64), ("head_dim", C.c_int64),
                ("cap", C.c_int64), ("stride_b", C.c_int64), ("stride_h", C.c_int64),
                ("stride_t", C.c_int64), ("dtype", C.c_int64)]


class LayerDesc(C.Structure):
    _fields_ = [("wqkv", C.c_void_p), ("wo", C.c_void_p), ("wgu", C.c_void_p), ("wd", C.c_void_p),
                ("attn_norm", C.c_void_p), ("ffn_norm", C.c_void_p), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("n_kv_heads", C.c_int64), ("head_dim", C.c_int64), ("cap", C.c_int64),
                ("window", C.c_int64), ("rope_theta", C.c_double), ("attn_scale", C.c_float),
                ("v_from_k", C.c_int32), ("kv_dtype", C.c_int32), ("rope_dims", C.c_int64),
                ("post_attn_norm", C.c_void_p), ("post_ffn_norm", C.c_void_p)]


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int64), ("d_model", C.c_int64), ("n_q_heads", C.c_int64),
                ("ffn", C.c_int64), ("vocab", C.c_int64), ("batch", C.c_int64),
                ("eps", C.c_float), ("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(LayerDesc)), ("ffn_act", C.c_int32),
                ("embed_scale", C.c_float), ("logit_softcap", C.c_float)]


_P, _I64, _F, _D, _SZ = C.c_void_p, C.c_int64, C.c_float, C.c_double, C.c_size_t
_SIGS = {
    "q4dec_last_error": ([], C.c_char_p),
    "q4dec_version": ([], C.c_char_p),
    "q4_0_matvec": ([_P, _I64, _I64, _P, _I64, _P, _P, _P], C.c_int),
    "q8_0_matvec": ([_P, _I64, _I64, _P, _I64, _P, _P, _P], C.c_int),
    "q8_0_gather": ([_P, _I64, _I64, _P, _I64, _P, _P], C.c_int),
    "q8_0_gather_scaled": ([_P, _I64, _I64, _P, _I64, _F, _P, _P], C.c_int),
    "q4_0_matvec_fused": ([_P, _I64, _I64, _P, _P, _I64, _I64, C.c_int, C.c_int, _P, _F, _P, _P, _P],
                          C.c_int),
    "q8_0_matvec_fused": ([_P, _I64, _I64, _P, _P, _I64, _I64, C.c_int, C.c_int, _P, _F, _P, _P, _P],
                          C.c_int),
    "q4_0_matvec_post_norm": ([_P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _F, _P, C.c_int, _P, _P],
                              C.c_int),
    "matvec_batched_workspace": ([_I64, _I64, _I64], _SZ),
    "q4_0_matvec_batched": ([_P, _I64, _I64, _P, _P, _I64, _I64, C.c_int, C.c_int, _P, _F, _P, _P,
                             _P, _SZ, _P], C.c_int),
    "q8_0_matvec_batched": ([_P, _I64, _I64, _P, _P, _I64, _I64, C.c_int, C.c_int, _P, _F, _P, _P,
                             _P, _SZ, _P], C.c_int),
    "q4_0_matvec_batched_noalloc": ([_P, _I64, _I64, _P, _P, _I64, _I64, C.c_int, C.c_int, _P, _F,
                                     _P, _P, _P], C.c_int),
    "rmsnorm": ([_P, _P, _I64, _I64, _F, _P, _P], C.c_int),
    "swiglu": ([_P, _P, _I64, _I64, _I64, _P, _P], C.c_int),
    "geglu": ([_P, _P, _I64, _I64, _I64, _P, _P], C.c_int),
    "rmsnorm_add": ([_P, _P, _I64, _I64, _F, _P, _P], C.c_int),
    "softcap": ([_P, _I64, _F, _P], C.c_int),
    "qk_norm_rope_partial": ([_P, _I64, _P, _P, _I64, _P, _P, _I64, C.POINTER(KVLayout), _P, _D,
                              _F, C.c_int, _I64, _P, _P, _P], C.c_int),
    "qk_norm_rope": ([_P, _I64, _P, _P, _I64, _P, _P, _I64, C.POINTER(KVLayout), _P, _D, _F,
                      C.c_int, _P, _P, _P], C.c_int),
    "gqa_decode_attn": ([_P, _I64, _I64, _P, _P, C.POINTER(KVLayout), _P, _I64, _F, _P, _I64,
                         _P, _SZ, _P], C.c_int),
    "gqa_decode_attn_workspace": ([C.POINTER(KVLayout), _I64, _I64], _SZ),
    "gqa_decode_attn_rope": ([_P, _I64, _I64, _P, _P, C.POINTER(KVLayout), _P, _D, _F, C.c_int, _P,
                              _P, _I64, _F, _P, _I64, _P, _SZ, _P], C.c_int),
    "argmax_rows": ([_P, _I64, _I64, _P, _P], C.c_int),
    "argmax_rows_workspace": ([_I64], _SZ),
    "argmax_rows_ws": ([_P, _I64, _I64, _P, _P, _SZ, _P], C.c_int),
    "decode_model_workspace": ([C.POINTER(ModelDesc), C.POINTER(_SZ)], C.c_int),
    "decode_model_create": ([C.POINTER(ModelDesc), _P, _SZ, C.POINTER(_P)], C.c_int),
    "decode_model_set_position": ([_P, _I64, _P], C.c_int),
    "decode_model_position": ([_P], _I64),
    "decode_step": ([_P, _P, _P, _P, _P], C.c_int),
    "decode_step_eager": ([_P, _P, _P, _P, _P], C.c_int),
    "decode_model_destroy": ([_P], C.c_int),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m q4_quantized_matvec_amd.build` (no CPU fallback exists)")
        _lib = _Bound(C.CDLL(LIB_PATH))
    return _lib


class _Bound:
    """Library wrapper that attaches the C signature to each symbol on first use."""

    def __init__(self, cdll):
        self._cdll = cdll

    def __getattr__(self, name):
        fn = getattr(self._cdll, name)  # AttributeError if the symbol is not exported
        if name in _SIGS:
            fn.argtypes, fn.restype = _SIGS[name]
        setattr(self, name, fn)
        return fn


def version() -> str:
    return lib().q4dec_version().decode()


def _check(name, status):
    if status != 0:
        raise Q4Error(name, status, lib().q4dec_last_error().decode())


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _cuda_f32(t, name):
    if t is None:
        return
    if not t.is_cuda or str(t.dtype) != "torch.float32":
        raise TypeError(f"{name} must be a float32 CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _qmatrix_dims(W, K, bpb):
    if not W.is_cuda or str(W.dtype) != "torch.uint8" or not W.is_contiguous():
        raise TypeError("W must be a contiguous uint8 CUDA tensor")
    row_bytes = K // 32 * bpb
    if row_bytes == 0 or W.numel() % row_bytes:
        raise ValueError("W size is not a whole number of rows")
    return W.numel() // row_bytes


def _matvec(name, bpb, W, x, y, residual, stream, n):
    import torch
    _cuda_f32(x, "x")
    B, K = (1, x.numel()) if x.dim() == 1 else x.shape
    N = n if n is not None else _qmatrix_dims(W, K, bpb)
    if y is None:
        y = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _cuda_f32(y, "y")
    _cuda_f32(residual, "residual")
    _check(name, getattr(lib(), name)(_ptr(W), N, K, _ptr(x), B, _ptr(y), _ptr(residual),
                                      _stream(stream)))
    return y


def q4_0_matvec(W, x, y=None, residual=None, stream=None, n=None):
    """y[B,N] = dequant(W) @ x[B,K] (+ residual).  W: uint8 [N, K/32*18] on device."""
    return _matvec("q4_0_matvec", 18, W, x, y, residual, stream, n)


def q8_0_matvec(W, x, y=None, residual=None, stream=None, n=None):
    """y[B,N] = dequant(W) @ x[B,K] (+ residual).  W: uint8 [N, K/32*34] on device."""
    return _matvec("q8_0_matvec", 34, W, x, y, residual, stream, n)


IN_PLAIN, IN_RMSNORM, IN_SWIGLU, IN_GEGLU = 0, 1, 2, 3
OUT_PLAIN, OUT_SWIGLU, OUT_GEGLU = 0, 1, 2


def _out_cols(N, out_op):
    return N // 2 if out_op in (OUT_SWIGLU, OUT_GEGLU) else N


def _matvec_fused(name, bpb, W, x, K, B, ld, op, x2, norm_w, eps, y, residual, stream, n, out_op):
    import torch
    N = n if n is not None else _qmatrix_dims(W, K, bpb)
    if y is None:
        y = torch.empty((B, _out_cols(N, out_op)), dtype=torch.float32, device=x.device)
    _check(name, getattr(lib(), name)(_ptr(W), N, K, _ptr(x), _ptr(x2), ld, B, int(op),
                                      int(out_op), _ptr(norm_w), float(eps), _ptr(y),
                                      _ptr(residual), _stream(stream)))
    return y


def q4_0_matvec_fused(W, x, K, B, ld, op, x2=None, norm_w=None, eps=0.0, y=None, residual=None,
                      stream=None, n=None, out_op=OUT_PLAIN):
    """y = out_op(dequant(W) @ op(x rows)) (+ residual); rows of x (and x2) at stride ld."""
    return _matvec_fused("q4_0_matvec_fused", 18, W, x, K, B, ld, op, x2, norm_w, eps, y,
                         residual, stream, n, out_op)


def q8_0_matvec_fused(W, x, K, B, ld, op, x2=None, norm_w=None, eps=0.0, y=None, residual=None,
                      stream=None, n=None, out_op=OUT_PLAIN):
    return _matvec_fused("q8_0_matvec_fused", 34, W, x, K, B, ld, op, x2, norm_w, eps, y,
                         residual, stream, n, out_op)


def q4_0_matvec_post_norm(W, h, z, K, B, ld, post_w, pre_w, eps, h_out, y=None, stream=None,
                          n=None, out_op=OUT_PLAIN):
    """h_out = h + post_w * rmsnorm(z); y = out_op(dequant(W) @ (pre_w * rmsnorm(h_out)));
    rows of h, z and h_out at stride ld."""
    import torch
    N = n if n is not None else _qmatrix_dims(W, K, 18)
    if y is None:
        y = torch.empty((B, _out_cols(N, out_op)), dtype=torch.float32, device=h.device)
    _check("q4_0_matvec_post_norm", lib().q4_0_matvec_post_norm(
        _ptr(W), N, K, _ptr(h), _ptr(z), ld, B, _ptr(post_w), _ptr(pre_w), float(eps), _ptr(h_out),
        int(out_op), _ptr(y), _stream(stream)))
    return y


def matvec_batched_workspace(N, K, B):
    """Bytes of device workspace q4_0/q8_0_matvec_batched need (0: shape unsupported)."""
    return int(lib().matvec_batched_workspace(N, K, B))


def _matvec_batched(name, bpb, W, x, K, B, ld, op, x2, norm_w, eps, y, residual, ws, stream, n,
                    out_op):
    import torch
    N = n if n is not None else _qmatrix_dims(W, K, bpb)
    if y is None:
        y = torch.empty((B, _out_cols(N, out_op)), dtype=torch.float32, device=x.device)
    if ws is None:  # split tickets must start at zero
        ws = torch.zeros(max(256, matvec_batched_workspace(N, K, B)), dtype=torch.uint8,
                         device=x.device)
    _check(name, getattr(lib(), name)(_ptr(W), N, K, _ptr(x), _ptr(x2), ld, B, int(op),
                                      int(out_op), _ptr(norm_w), float(eps), _ptr(y),
                                      _ptr(residual), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def q4_0_matvec_batched(W, x, K, B, ld, op=0, x2=None, norm_w=None, eps=0.0, y=None,
                        residual=None, ws=None, stream=None, n=None, out_op=OUT_PLAIN):
    """As q4_0_matvec_fused, on the matrix cores (1 <= B <= 32, K % 256 == 0).  ``ws``: a
    zero-initialised uint8 device tensor of matvec_batched_workspace(N, K, B) bytes, reusable
    across calls on one stream (allocated if None)."""
    return _matvec_batched("q4_0_matvec_batched", 18, W, x, K, B, ld, op, x2, norm_w, eps, y,
                           residual, ws, stream, n, out_op)


def q8_0_matvec_batched(W, x, K, B, ld, op=0, x2=None, norm_w=None, eps=0.0, y=None,
                        residual=None, ws=None, stream=None, n=None, out_op=OUT_PLAIN):
    return _matvec_batched("q8_0_matvec_batched", 34, W, x, K, B, ld, op, x2, norm_w, eps, y,
                           residual, ws, stream, n, out_op)


NOALLOC_SCRATCH_BYTES = 16 << 20  # Q4_NOALLOC_SCRATCH_BYTES


def q4_0_matvec_batched_noalloc(W, x, K, B, ld, op=0, x2=None, norm_w=None, eps=0.0, y=None,
                                residual=None, stream=None, n=None, out_op=OUT_PLAIN):
    """q4_0_matvec_batched with its scratch in the library's static per-device array
    (no workspace argument; the library allocates nothing).  Pass ``y`` to avoid the
    output allocation on the Python side."""
    import torch
    N = n if n is not None else _qmatrix_dims(W, K, 18)
    if y is None:
        y = torch.empty((B, _out_cols(N, out_op)), dtype=torch.float32, device=x.device)
    _check("q4_0_matvec_batched_noalloc", lib().q4_0_matvec_batched_noalloc(
        _ptr(W), N, K, _ptr(x), _ptr(x2), ld, B, int(op), int(out_op), _ptr(norm_w), float(eps),
        _ptr(y), _ptr(residual), _stream(stream)))
    return y


def q8_0_gather(E, tokens, K, x=None, stream=None, scale=None):
    """Rows tokens of the Q8_0 table E dequantised (times scale if given)."""
    import torch
    V = _qmatrix_dims(E, K, 34)
    B = tokens.numel()
    if x is None:
        x = torch.empty((B, K), dtype=torch.float32, device=tokens.device)
    if scale is None:
        _check("q8_0_gather", lib().q8_0_gather(_ptr(E), V, K, _ptr(tokens), B, _ptr(x),
                                                _stream(stream)))
    else:
        _check("q8_0_gather_scaled", lib().q8_0_gather_scaled(_ptr(E), V, K, _ptr(tokens), B,
                                                              float(scale), _ptr(x),
                                                              _stream(stream)))
    return x


def rmsnorm(x, w, eps, y=None, stream=None):
    import torch
    _cuda_f32(x, "x")
    dim = x.shape[-1]
    rows = x.numel() // dim
    if y is None:
        y = torch.empty_like(x)
    _check("rmsnorm", lib().rmsnorm(_ptr(x), _ptr(w), rows, dim, eps, _ptr(y), _stream(stream)))
    return y


def swiglu(g, u, rows, n, ld, h=None, stream=None):
    """h[rows, n] = silu(g) * u, g/u read with row stride ld (elements)."""
    import torch
    if h is None:
        h = torch.empty((rows, n), dtype=torch.float32, device=g.device)
    _check("swiglu", lib().swiglu(_ptr(g), _ptr(u), rows, n, ld, _ptr(h), _stream(stream)))
    return h


def geglu(g, u, rows, n, ld, h=None, stream=None):
    """h[rows, n] = gelu(g) * u (tanh form), g/u read with row stride ld."""
    import torch
    if h is None:
        h = torch.empty((rows, n), dtype=torch.float32, device=g.device)
    _check("geglu", lib().geglu(_ptr(g), _ptr(u), rows, n, ld, _ptr(h), _stream(stream)))
    return h


def rmsnorm_add(y, w, eps, x, stream=None):
    """x += w * y / rms(y), row by row (the last axis)."""
    _cuda_f32(y, "y")
    dim = y.shape[-1]
    rows = y.numel() // dim
    _check("rmsnorm_add", lib().rmsnorm_add(_ptr(y), _ptr(w), rows, dim, eps, _ptr(x),
                                            _stream(stream)))
    return x


def softcap(v, cap, stream=None):
    """v = cap * tanh(v / cap) in place."""
    _check("softcap", lib().softcap(_ptr(v), v.numel(), float(cap), _stream(stream)))
    return v


def kv_dtype_of(cache):
    import torch
    if cache.dtype == torch.float32:
        return KV_F32
    if cache.dtype == torch.float16:
        return KV_F16
    raise TypeError(f"KV cache dtype {cache.dtype} is neither float32 nor float16")


def kv_layout_of(cache):
    """Layout of a cache tensor [B, Hkv, cap, hd] (float32 or float16, hd contiguous)."""
    B, H, cap, hd = cache.shape
    s = cache.stride()
    return KVLayout(B, H, hd, cap, s[0], s[1], s[2], kv_dtype_of(cache))


def qk_norm_rope(q, ldq, k, v, ldkv, q_norm, k_norm, n_q_heads, kv, pos_dev, theta, eps,
                 v_from_k, k_cache, v_cache, stream=None, rot_dims=None):
    """rot_dims (p-RoPE): rotate only the first rot_dims elements of each head."""
    if rot_dims is None:
        _check("qk_norm_rope", lib().qk_norm_rope(
            _ptr(q), ldq, _ptr(k), _ptr(v), ldkv, _ptr(q_norm), _ptr(k_norm), n_q_heads,
            C.byref(kv), _ptr(pos_dev), float(theta), float(eps), int(bool(v_from_k)),
            _ptr(k_cache), _ptr(v_cache), _stream(stream)))
    else:
        _check("qk_norm_rope_partial", lib().qk_norm_rope_partial(
            _ptr(q), ldq, _ptr(k), _ptr(v), ldkv, _ptr(q_norm), _ptr(k_norm), n_q_heads,
            C.byref(kv), _ptr(pos_dev), float(theta), float(eps), int(bool(v_from_k)),
            int(rot_dims), _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def gqa_decode_attn_workspace(kv, n_q_heads, window):
    return lib().gqa_decode_attn_workspace(C.byref(kv), n_q_heads, window)


def gqa_decode_attn(q, ldq, n_q_heads, k_cache, v_cache, kv, n_dev, window, scale, out, ldo,
                    ws, stream=None):
    _check("gqa_decode_attn", lib().gqa_decode_attn(
        _ptr(q), ldq, n_q_heads, _ptr(k_cache), _ptr(v_cache), C.byref(kv), _ptr(n_dev),
        int(window), float(scale), _ptr(out), ldo, _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def gqa_decode_attn_rope(qkv, ld, n_q_heads, q_norm, k_norm, kv, pos_dev, theta, eps, v_from_k,
                         k_cache, v_cache, window, scale, out, ldo, ws, stream=None):
    """QK-norm + RoPE + KV append + attention in one call (q, k, v read raw from qkv rows)."""
    _check("gqa_decode_attn_rope", lib().gqa_decode_attn_rope(
        _ptr(qkv), ld, n_q_heads, _ptr(q_norm), _ptr(k_norm), C.byref(kv), _ptr(pos_dev),
        float(theta), float(eps), int(bool(v_from_k)), _ptr(k_cache), _ptr(v_cache), int(window),
        float(scale), _ptr(out), ldo, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def argmax_rows(logits, out=None, stream=None):
    import torch
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check("argmax_rows", lib().argmax_rows(_ptr(logits), B, V, _ptr(out), _stream(stream)))
    return out


def argmax_rows_ws(logits, out=None, ws=None, stream=None):
    """argmax_rows in two passes (64 workgroups per row) with a workspace."""
    import torch
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    if ws is None:
        ws = torch.empty(lib().argmax_rows_workspace(B), dtype=torch.uint8, device=logits.device)
    _check("argmax_rows_ws", lib().argmax_rows_ws(_ptr(logits), B, V, _ptr(out), _ptr(ws),
                                                  ws.numel(), _stream(stream)))
    return out


class DecodeModel:
    """Host handle of a resident decode model (weights/caches stay caller-owned).

    ``layers``: list of dicts with device tensors wqkv, wo, wgu, wd, attn_norm,
    ffn_norm, q_norm, k_norm, k_cache, v_cache and ints/floats n_kv_heads,
    head_dim, window, rope_theta, attn_scale, v_from_k; optionally rope_dims
    (p-RoPE) and post_attn_norm / post_ffn_norm tensors (sandwich norms).
    ``ffn_act`` ("silu" or "gelu_tanh"), ``embed_scale`` and ``logit_softcap``
    select the Gemma-4 block variants (defaults: off).
    """

    def __init__(self, *, d_model, n_q_heads, ffn, vocab, batch, eps, embed, final_norm,
                 layers, device=None, ffn_act="silu", embed_scale=0.0, logit_softcap=0.0):
        import torch
        self._keep = [embed, final_norm]
        arr = (LayerDesc * len(layers))()
        for i, L in enumerate(layers):
            d = arr[i]
            for key in ("wqkv", "wo", "wgu", "wd", "attn_norm", "ffn_norm", "q_norm", "k_norm",
                        "k_cache", "v_cache"):
                setattr(d, key, _ptr(L[key]))
                self._keep.append(L[key])
            d.n_kv_heads = L["n_kv_heads"]
            d.head_dim = L["head_dim"]
            d.cap = L["k_cache"].shape[2]
            d.window = L["window"]
            d.rope_theta = L["rope_theta"]
            d.attn_scale = L["attn_scale"]
            d.v_from_k = 1 if L["v_from_k"] else 0
            d.kv_dtype = kv_dtype_of(L["k_cache"])
            if kv_dtype_of(L["v_cache"]) != d.kv_dtype:
                raise TypeError(f"layer {i}: k_cache and v_cache dtypes differ")
            d.rope_dims = int(L.get("rope_dims", 0) or 0)
            for key in ("post_attn_norm", "post_ffn_norm"):
                if L.get(key) is not None:
                    _cuda_f32(L[key], key)
                    setattr(d, key, _ptr(L[key]))
                    self._keep.append(L[key])
        self._layers = arr
        acts = {"silu": 0, "gelu_tanh": 1}
        if ffn_act not in acts:
            raise ValueError(f"ffn_act {ffn_act!r} is neither 'silu' nor 'gelu_tanh'")
        desc = ModelDesc(len(layers), d_model, n_q_heads, ffn, vocab, batch, eps, _ptr(embed),
                         _ptr(final_norm), C.cast(arr, C.POINTER(LayerDesc)), acts[ffn_act],
                         float(embed_scale or 0.0), float(logit_softcap or 0.0))
        self._desc = desc
        nbytes = C.c_size_t()
        _check("decode_model_workspace", lib().decode_model_workspace(C.byref(desc),
                                                                      C.byref(nbytes)))
        dev = device or embed.device
        self.workspace = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
        h = C.c_void_p()
        _check("decode_model_create", lib().decode_model_create(
            C.byref(desc), _ptr(self.workspace), nbytes.value, C.byref(h)))
        self._h = h
        self.batch, self.vocab = batch, vocab

    def set_position(self, pos, stream=None):
        _check("decode_model_set_position",
               lib().decode_model_set_position(self._h, int(pos), _stream(stream)))

    @property
    def position(self):
        return lib().decode_model_position(self._h)

    def step(self, tokens, next_tokens, logits=None, stream=None, eager=False):
        fn = lib().decode_step_eager if eager else lib().decode_step
        _check("decode_step", fn(self._h, _ptr(tokens), _ptr(next_tokens), _ptr(logits),
                                 _stream(stream)))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().decode_model_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
