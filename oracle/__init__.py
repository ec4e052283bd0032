"""CPU oracle for the paged BF16 block operator -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never imports, links or calls it, and it never imports the product.

The arithmetic lives in ``psi_oracle.c`` (plain C, dense, fp32 sequential
accumulation, declared BF16 write boundaries); this module only marshals
numpy arrays.  BF16 values are passed as ``numpy.uint16`` bit patterns.

Citations [PSI] refer to "Precision-Preserving Subtensor Inference for a 22B
Joint Audio-Video Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("PSI_ORACLE_LIB")  # a mutated build, for the pin self-test
    path = override or _build.LIB
    if not override and (not os.path.exists(path)
                         or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
        _build.build()
    _lib = _configure(ctypes.CDLL(path))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every oracle call through another build of
    ``psi_oracle.c`` (the tests use this to check that the pins reject
    deliberately mutated copies of the oracle)."""
    global _lib
    saved = _load()
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _configure(lib):
    lib.orc_threads.restype = ctypes.c_int
    lib.orc_threads.argtypes = []
    lib.orc_f.restype = ctypes.c_float
    lib.orc_f.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_from_float.restype = ctypes.c_uint16
    lib.orc_bf16_from_float.argtypes = [ctypes.c_float]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
    lib.orc_gelu_tanh_double.restype = ctypes.c_double
    lib.orc_gelu_tanh_double.argtypes = [ctypes.c_double]
    lib.orc_gelu_bf16.restype = None
    lib.orc_gelu_bf16.argtypes = [_u16p, ctypes.c_size_t, _u16p]
    lib.orc_linear.restype = None
    lib.orc_linear.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int,
                               _u16p, ctypes.c_int, _f32p, _f32p, _u16p]
    lib.orc_ffn.restype = ctypes.c_int
    lib.orc_ffn.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int, _u16p,
                            _u16p, ctypes.c_int, _u16p, ctypes.c_int, ctypes.c_int,
                            _u16p, _f32p, _u16p]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_attention.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, _u16p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _u16p, ctypes.c_int]
    lib.orc_attn_sublayer.restype = ctypes.c_int
    lib.orc_attn_sublayer.argtypes = [_u16p, ctypes.c_int, _u16p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p,
                                      ctypes.c_int, ctypes.c_int, _u16p, _f32p, _u16p]
    lib.orc_block.restype = ctypes.c_int
    lib.orc_block.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int] + [_u16p] * 12 + [ctypes.c_int]
    lib.orc_attention_ex.restype = ctypes.c_int
    lib.orc_attention_ex.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, _u16p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _u16p, ctypes.c_int]
    lib.orc_rmsnorm.restype = None
    lib.orc_rmsnorm.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_double,
                                ctypes.c_int, _u16p, ctypes.c_int]
    lib.orc_rope_split.restype = None
    lib.orc_rope_split.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p,
                                   _f32p, _u16p, ctypes.c_int]
    lib.orc_attn_sublayer_ext.restype = ctypes.c_int
    lib.orc_attn_sublayer_ext.argtypes = [_u16p, ctypes.c_int, _u16p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int] + [_u16p] * 10 + \
        [ctypes.c_double, ctypes.c_int, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
         ctypes.c_int, _u16p]
    lib.orc_residual.restype = None
    lib.orc_residual.argtypes = [_u16p, _u16p, ctypes.c_size_t]
    return lib


def _u16(a, name="array"):
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.dtype == np.uint16 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous numpy uint16 (bf16 bits) array")
    return a.ctypes.data_as(_u16p)


def _f32(a, name="array"):
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.dtype == np.float32 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous numpy float32 array")
    return a.ctypes.data_as(_f32p)


# ---------------------------------------------------------------- scalars

def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().orc_threads())


def bf16_to_float(u) -> np.ndarray:
    """f(): widen bf16 bit patterns to float32 (exact)."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_from_float_scalar(v: float) -> int:
    """B() of one binary32 value, evaluated by the C oracle."""
    return int(_load().orc_bf16_from_float(ctypes.c_float(v)))


def bf16_from_double_scalar(v: float) -> int:
    """B() of one double, rounded once, evaluated by the C oracle."""
    return int(_load().orc_bf16_from_double(ctypes.c_double(v)))


def gelu_tanh_double(v: float) -> float:
    return float(_load().orc_gelu_tanh_double(ctypes.c_double(v)))


def gelu_bf16(u: np.ndarray) -> np.ndarray:
    """H = B(phi(f(u))) elementwise, [PSI] sec. II-B eq. (2) with sec. III-A's
    BF16 write after GELU."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    h = np.empty_like(u)
    _load().orc_gelu_bf16(_u16(u), u.size, _u16(h))
    return h


# ---------------------------------------------------------------- operators

def linear(x, W, b=None, *, variant=0, acc_in=None, want_acc=False):
    """y = B(x W^T + b) with fp32 sequential accumulation ([PSI] sec. III-A).

    Returns y (uint16 [M,N]), or (y, acc) when ``want_acc``; ``acc_in``
    continues a carried fp32 chain (K-split partition, [PSI] sec. II-B)."""
    M, K = x.shape
    N, K2 = W.shape
    assert K == K2
    y = np.empty((M, N), dtype=np.uint16)
    acc = np.empty((M, N), dtype=np.float32) if want_acc else None
    if b is not None:
        assert b.shape == (N,)
    if acc_in is not None:
        assert acc_in.shape == (M, N)
    _load().orc_linear(_u16(x, "x"), M, K, _u16(W, "W"), N, _u16(b, "b"), int(variant),
                       _f32(acc_in, "acc_in"), _f32(acc, "acc"), _u16(y))
    return (y, acc) if want_acc else y


def ffn(x, U, a, V, b, *, variant=0, residual=False, want_hidden=False, want_acc=False):
    """Dense FFN F(X) = phi(X U^T + a) V^T + b with [PSI] sec. III-A's BF16
    boundaries; optional residual y = B(x + F(x))."""
    M, d = x.shape
    h, d2 = U.shape
    r, h2 = V.shape
    assert d == d2 and h == h2 and a.shape == (h,) and b.shape == (r,)
    y = np.empty((M, r), dtype=np.uint16)
    H = np.empty((M, h), dtype=np.uint16) if want_hidden else None
    acc = np.empty((M, r), dtype=np.float32) if want_acc else None
    rc = _load().orc_ffn(_u16(x), M, d, _u16(U), h, _u16(a), _u16(V), r, _u16(b),
                         int(variant), int(bool(residual)), _u16(H), _f32(acc), _u16(y))
    if rc != 0:
        raise RuntimeError(f"orc_ffn failed: {rc}")
    out = [y]
    if want_hidden:
        out.append(H)
    if want_acc:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def attention(q, k, v, heads, dh):
    """Dense per-head softmax attention ([PSI] eq. (3) over all keys) with
    fp32 weights; q [Mq, heads*dh], k/v [Mk, heads*dh] -> o [Mq, heads*dh]."""
    Mq, dq = q.shape
    Mk, dk = k.shape
    assert v.shape == (Mk, dk) and dq == dk == heads * dh
    o = np.empty((Mq, dq), dtype=np.uint16)
    rc = _load().orc_attention(_u16(q), Mq, dq, _u16(k), _u16(v), Mk, dk, dk, heads, dh,
                               _u16(o), dq)
    if rc != 0:
        raise RuntimeError(f"orc_attention failed: {rc}")
    return o


def attn_sublayer(x, Wq, bq, Wk, bk, Wv, bv, Wo, bo, heads, dh, *, ctx=None, variant=0,
                  residual=True, want_o=False, want_acc=False):
    M, d = x.shape
    Mc = 0 if ctx is None else ctx.shape[0]
    y = np.empty((M, d), dtype=np.uint16)
    O = np.empty((M, d), dtype=np.uint16) if want_o else None
    acc = np.empty((M, d), dtype=np.float32) if want_acc else None
    rc = _load().orc_attn_sublayer(_u16(x), M, _u16(ctx), Mc, d, heads, dh,
                                   _u16(Wq), _u16(bq), _u16(Wk), _u16(bk), _u16(Wv), _u16(bv),
                                   _u16(Wo), _u16(bo), int(variant), int(bool(residual)),
                                   _u16(O), _f32(acc), _u16(y))
    if rc != 0:
        raise RuntimeError(f"orc_attn_sublayer failed: {rc}")
    out = [y]
    if want_o:
        out.append(O)
    if want_acc:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def block(x, w, heads, dh, *, variant=0):
    """One synthetic block (self-attention sub-block then FFN sub-block, each
    with residual).  ``w`` maps Wq,bq,Wk,bk,Wv,bv,Wo,bo,U,a,V,b to arrays.
    Returns the new x (a copy)."""
    x = np.array(x, dtype=np.uint16, copy=True, order="C")
    M, d = x.shape
    hidden = w["U"].shape[0]
    names = ["Wq", "bq", "Wk", "bk", "Wv", "bv", "Wo", "bo", "U", "a", "V", "b"]
    rc = _load().orc_block(_u16(x), M, d, heads, dh, hidden, *[_u16(w[n], n) for n in names],
                           int(variant))
    if rc != 0:
        raise RuntimeError(f"orc_block failed: {rc}")
    return x


def residual(x, y):
    out = np.array(x, dtype=np.uint16, copy=True, order="C")
    _load().orc_residual(_u16(out), _u16(np.ascontiguousarray(y, dtype=np.uint16)), out.size)
    return out


def attention_ex(q, k, v, heads, dh, *, bf16_p=False):
    """orc_attention with the baseline BF16-numerator choice (bf16_p)."""
    Mq, dq = q.shape
    Mk, dk = k.shape
    assert v.shape == (Mk, dk) and dq == dk == heads * dh
    o = np.empty((Mq, dq), dtype=np.uint16)
    rc = _load().orc_attention_ex(_u16(q), Mq, dq, _u16(k), _u16(v), Mk, dk, dk, heads, dh,
                                  int(bool(bf16_p)), _u16(o), dq)
    if rc != 0:
        raise RuntimeError(f"orc_attention_ex failed: {rc}")
    return o


def rmsnorm(x, g, eps=1e-6, tile=0):
    """Full-row RMS normalisation with a tile-partitioned sum of squares."""
    M, d = x.shape
    y = np.empty((M, d), dtype=np.uint16)
    _load().orc_rmsnorm(_u16(x), M, d, d, _u16(g), float(eps), int(tile), _u16(y), d)
    return y


def rope_split(x, heads, dh, cos, sin):
    """Split rotary embedding per head with fp32 tables [M, dh/2]."""
    M, d = x.shape
    assert d == heads * dh and cos.shape == sin.shape == (M, dh // 2)
    y = np.empty((M, d), dtype=np.uint16)
    _load().orc_rope_split(_u16(x), M, heads, dh, d, _f32(cos), _f32(sin), _u16(y), d)
    return y


def attn_sublayer_ext(x, w, heads, dh, *, ctx=None, gq=None, gk=None, eps=1e-6, norm_tile=0,
                      cos_q=None, sin_q=None, cos_k=None, sin_k=None, variant=0, bf16_p=False,
                      residual=True):
    """Attention sub-block with optional q/k RMS normalisation and split
    rotary positions; ``w`` maps Wq,bq,Wk,bk,Wv,bv,Wo,bo to arrays."""
    M, d = x.shape
    Mc = 0 if ctx is None else ctx.shape[0]
    y = np.empty((M, d), dtype=np.uint16)
    names = ["Wq", "bq", "Wk", "bk", "Wv", "bv", "Wo", "bo"]
    rc = _load().orc_attn_sublayer_ext(_u16(x), M, _u16(ctx), Mc, d, heads, dh,
                                       *[_u16(w[n], n) for n in names], _u16(gq), _u16(gk),
                                       float(eps), int(norm_tile), _f32(cos_q), _f32(sin_q),
                                       _f32(cos_k), _f32(sin_k), int(variant), int(bool(bf16_p)),
                                       int(bool(residual)), _u16(y))
    if rc != 0:
        raise RuntimeError(f"orc_attn_sublayer_ext failed: {rc}")
    return y
