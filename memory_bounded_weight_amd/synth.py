"""Seeded synthetic inputs for the paged block operator.

This module holds no arithmetic of the method itself: it only draws seeded
normal numbers and stores them as bfloat16 bit patterns.  Both the HIP path
(through the tests and the benchmark) and the CPU oracle receive the SAME
bytes from here.

Recipe (the workloads of the paper are LTX-2.5 blocks whose checkpoint is
not available; random weights of the same shapes stand in):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64), draws with
    ``standard_normal(dtype=float32)`` in a fixed order;
  * ``N(0, v)`` means variance ``v``: the float32 draw is multiplied by the
    float32 value of sqrt(v), then rounded to bfloat16 (nearest, ties to
    even);
  * activations N(0, 1); weights N(0, 1/fan_in); biases N(0, 0.02);
  * a stack of blocks draws block ``i``'s weights from
    ``default_rng([seed, i])`` so one block can be regenerated alone;
  * normalisation gains gamma ~ 1 + N(0, 0.01) (the float32 sum, rounded
    to bfloat16);
  * rotary tables are the caller's inputs: for token position t and pair
    index j < dh/2, the angle t * base^(-2j/dh) (base 10000) in float64,
    cos and sin rounded to float32.
"""
from __future__ import annotations

import math

import numpy as np

BIAS_VAR = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (nearest, ties to even).
    Inputs are finite draws; no NaN handling is needed here."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    w = a.view(np.uint32)
    lsb = (w >> np.uint32(16)) & np.uint32(1)
    return ((w + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(math.sqrt(var))
    return f32_to_bf16_bits(z)


def linear_weights(rng, n_out: int, n_in: int):
    """One Linear layer: W [n_out, n_in] ~ N(0, 1/n_in), b [n_out] ~ N(0, 0.02)."""
    W = normal_bf16(rng, (n_out, n_in), 1.0 / n_in)
    b = normal_bf16(rng, (n_out,), BIAS_VAR)
    return W, b


def linear_case(seed: int = 0, M: int = 64, K: int = 256, N: int = 512):
    """Single paged linear: x [M,K] ~ N(0,1), W [N,K] ~ N(0,1/K), b [N] ~ N(0,0.02).
    The default sizes are the 64 x 256 -> 512 parity case."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, K), 1.0)
    W = normal_bf16(rng, (N, K), 1.0 / K)
    b = normal_bf16(rng, (N,), BIAS_VAR)
    return {"x": x, "W": W, "b": b}


def ffn_case(seed: int = 0, M: int = 1024, d: int = 2048, hidden: int = 8192):
    """FFN: x [M,d] ~ N(0,1); U [hidden,d] ~ N(0,1/d), a [hidden];
    V [d,hidden] ~ N(0,1/hidden), b [d]."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, d), 1.0)
    U, a = linear_weights(rng, hidden, d)
    V, b = linear_weights(rng, d, hidden)
    return {"x": x, "U": U, "a": a, "V": V, "b": b}


def attn_weights(rng, d: int):
    out = {}
    for n in ("q", "k", "v", "o"):
        W, b = linear_weights(rng, d, d)
        out["W" + n] = W
        out["b" + n] = b
    return out


def attn_case(seed: int = 0, M: int = 6144, Mc: int = 1024, d: int = 4096, cross: bool = True):
    """Attention sub-blocks: x [M,d] ~ N(0,1), ctx [Mc,d] ~ N(0,1), then the
    self-attention Wq,bq,Wk,bk,Wv,bv,Wo,bo and (if ``cross``) the
    cross-attention ones, each W ~ N(0,1/d)."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, d), 1.0)
    ctx = normal_bf16(rng, (Mc, d), 1.0) if cross else None
    self_w = attn_weights(rng, d)
    cross_w = attn_weights(rng, d) if cross else None
    return {"x": x, "ctx": ctx, "self": self_w, "cross": cross_w}


def block_weights(seed: int, index: int, d: int = 4096, hidden: int = 16384):
    """Weights of block ``index`` of a synthetic stack: attention
    Wq,bq,Wk,bk,Wv,bv,Wo,bo then FFN U,a,V,b."""
    rng = np.random.default_rng([seed, index])
    w = attn_weights(rng, d)
    w["U"], w["a"] = linear_weights(rng, hidden, d)
    w["V"], w["b"] = linear_weights(rng, d, hidden)
    return w


def stack_input(seed: int = 0, M: int = 8192, d: int = 4096):
    rng = np.random.default_rng(seed)
    return normal_bf16(rng, (M, d), 1.0)


def norm_gamma(rng, d: int) -> np.ndarray:
    z = rng.standard_normal(size=(d,), dtype=np.float32)
    return f32_to_bf16_bits(np.float32(1.0) + z * np.float32(0.1))


def rope_tables(M: int, dh: int, offset: int = 0, base: float = 10000.0):
    """cos/sin tables [M, dh/2] (float32) for positions offset .. offset+M-1."""
    t = np.arange(offset, offset + M, dtype=np.float64)[:, None]
    j = np.arange(dh // 2, dtype=np.float64)[None, :]
    ang = t * base ** (-2.0 * j / dh)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def attn_ext_case(seed: int = 0, M: int = 126, d: int = 2048, Mc: int = 0):
    """Attention sub-block with q/k normalisation and rotary positions; the
    defaults are the audio self-attention shape (126 tokens, d 2,048, which
    is 32 heads of 64).  x [M,d] ~ N(0,1), ctx [Mc,d] ~ N(0,1) when Mc > 0,
    the eight projection arrays as attn_weights, then gamma_q, gamma_k."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (M, d), 1.0)
    ctx = normal_bf16(rng, (Mc, d), 1.0) if Mc > 0 else None
    w = attn_weights(rng, d)
    gq = norm_gamma(rng, d)
    gk = norm_gamma(rng, d)
    return {"x": x, "ctx": ctx, "w": w, "gq": gq, "gk": gk}


def lattice_attn_case(seed: int = 0, M: int = 126, d: int = 2048):
    """Attention inputs on an integer lattice: x in {-2..2}, W in
    {-1, 0, 1}/64, biases in {-2..2}/64 (uniform draws).  Every product and
    partial sum of a projection is a multiple of 1/64 below 2^24/64 in
    magnitude, so the fp32 sum is exact in any order and the GPU and the
    oracle project to the same BF16 Q, K, V."""
    rng = np.random.default_rng(seed)
    lat = lambda shape, lo, hi, s: f32_to_bf16_bits(
        rng.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(s))
    x = lat((M, d), -2, 2, 1.0)
    w = {}
    for n in ("q", "k", "v", "o"):
        w["W" + n] = lat((d, d), -1, 1, 1.0 / 64)
        w["b" + n] = lat((d,), -2, 2, 1.0 / 64)
    return {"x": x, "w": w}
