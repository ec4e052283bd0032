"""GEMM epilogue: whole wave blocks and ragged ones give the same bits.

A wave block of the GEMM that lies wholly inside the output takes a
separate epilogue: scalar row addresses, the packed conversion
instruction for the BF16 rounding, with NaN made canonical before it.  Ragged
blocks keep the general epilogue.  Running an operator on M and on M - 1
tokens moves the rows of the last full wave block to the ragged path; the
shared rows must not change, NaN and infinities included, and every NaN
output must be the canonical 0x7FC0 that B() gives ([PSI] sec. III-A: the
BF16 rounding of each stored value).  Covered: output-column pages with bias
and residual, the K-split chain (fp32 accumulator loaded and stored), the
FFN (GELU epilogue, then the carried down-projection with residual), the
attention's K and transposed V projections (bias along columns and along
rows, on an integer lattice also against the oracle), for the 256 x 128 and
the 64 x 64 tile shapes.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import MiB, dev, empty_bf16, f, host, make_arena

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def with_specials(x, rows):
    """NaN of both signs, a signalling-pattern NaN and infinities in a few
    rows (an infinity times weights of both signs also makes inf - inf)."""
    x = x.copy()
    specials = [0x7FC0, 0xFFC1, 0x7F81, 0x7F80, 0xFF80]
    for k, r in enumerate(rows):
        x[r, (7 * k) % x.shape[1]] = specials[k % len(specials)]
    return x


def linear(P, x, W, b, split, block, flags):
    M, K = x.shape
    m = P.pinned_matrix(W, b, split, block)
    ar = make_arena(64 * MiB, W.shape[0] * W.shape[1] * 2, 2)
    try:
        y = empty_bf16(M, W.shape[0])
        acc = torch.zeros(M, W.shape[0], dtype=torch.float32, device="cuda")
        P.psi_linear_paged(ar, dev(x), M, K, m, acc, y, flags)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


def ffn(P, x, U, a_, V, b, tile):
    M, d = x.shape
    mu = P.pinned_matrix(U, a_, P.PSI_SPLIT_ROWS, tile)
    mv = P.pinned_matrix(V, b, P.PSI_SPLIT_COLS, tile)
    ar = make_arena(96 * MiB, tile * d * 2, 2)
    try:
        y = empty_bf16(M, d)
        acc = torch.zeros(M, d, dtype=torch.float32, device="cuda")
        P.psi_ffn_paged(ar, dev(x), M, d, mu, mv, 1, acc, y, P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


def check_same(full, ragged):
    n = ragged.shape[0]
    assert np.array_equal(full[:n], ragged)
    nan = np.isnan(f(full))
    assert nan.any(), "the case must produce NaN outputs"
    assert np.all(full[nan] == 0x7FC0), np.unique(full[nan])


# (M, d): 4224 x 1024 outputs take 256 x 128 workgroups (more than 256 tiles
# of 128 x 128); 512 x 256 take 64 x 64 ones.  M - 1 makes the last wave
# block of 64 (32) rows ragged.
SHAPES = [(4224, 1024, 64), (512, 256, 32)]


@pytest.mark.parametrize("M,d,wave_rows", SHAPES)
@pytest.mark.parametrize("split", ["rows", "cols"])
def test_linear_whole_and_ragged_blocks_same_bits(P, M, d, wave_rows, split):
    rng = np.random.default_rng(90 + d)
    x = synth.normal_bf16(rng, (M, d), 1.0)
    W = synth.normal_bf16(rng, (d, d), 1.0 / np.sqrt(d))
    b = synth.normal_bf16(rng, (d,), 0.1)
    edge = M - wave_rows  # first row of the last wave block
    x = with_specials(x, [5, 77, edge, edge + 3, edge + 9, M - 2])
    sp = P.PSI_SPLIT_ROWS if split == "rows" else P.PSI_SPLIT_COLS
    blk = d // 4
    full = linear(P, x, W, b, sp, blk, P.PSI_OP_RESIDUAL)
    ragged = linear(P, x[:M - 1], W, b, sp, blk, P.PSI_OP_RESIDUAL)
    check_same(full, ragged)
    # no residual: the plain bias epilogue
    full = linear(P, x, W, b, sp, blk, 0)
    ragged = linear(P, x[:M - 1], W, b, sp, blk, 0)
    check_same(full, ragged)


@pytest.mark.parametrize("M,d,wave_rows", SHAPES)
def test_ffn_whole_and_ragged_blocks_same_bits(P, M, d, wave_rows):
    rng = np.random.default_rng(95 + d)
    h = 4 * d
    x = synth.normal_bf16(rng, (M, d), 1.0)
    U = synth.normal_bf16(rng, (h, d), 1.0 / np.sqrt(d))
    a_ = synth.normal_bf16(rng, (h,), 0.1)
    V = synth.normal_bf16(rng, (d, h), 1.0 / np.sqrt(h))
    b = synth.normal_bf16(rng, (d,), 0.1)
    edge = M - wave_rows
    x = with_specials(x, [3, edge + 1, edge + 5, M - 3])
    full = ffn(P, x, U, a_, V, b, h // 4)
    ragged = ffn(P, x[:M - 1], U, a_, V, b, h // 4)
    check_same(full, ragged)


def lattice(rng, shape, lo, hi):
    """Small integers as bf16 bits: every product and sum of the GEMMs
    below is exact in fp32, so any summation order gives the same value."""
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return synth.f32_to_bf16_bits(v)


def attn_kv(P, x, w, heads, gw):
    """K_g and V_g^T of the last head group after psi_attn_paged with Wo in
    output tiles: they sit behind the [M, d] head-group outputs in the
    accumulator's memory (256-byte aligned, V^T rows padded to a multiple
    of 64 keys)."""
    M, d = x.shape
    ms = [P.pinned_matrix(w["W" + n], w["b" + n], P.PSI_SPLIT_ROWS, gw) for n in "qkv"]
    ms.append(P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_ROWS, gw))
    ar = make_arena(64 * MiB, gw * d * 2, 3)
    try:
        y = empty_bf16(M, d)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        P.psi_attn_paged(ar, dev(x), M, None, 0, heads, d // heads, *ms, acc, y, P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        raw = acc.cpu().numpy().view(np.uint16).reshape(-1)
    finally:
        P.psi_arena_destroy(ar)
    al = lambda n: (n + 255) // 256 * 256
    o16, k16 = al(M * d * 2) // 2, al(M * gw * 2) // 2
    ldvt = (M + 63) // 64 * 64
    K = raw[o16:o16 + M * gw].reshape(M, gw)
    Vt = raw[o16 + k16:o16 + k16 + gw * ldvt].reshape(gw, ldvt)[:, :M]
    return K, Vt


# (M, d, head-group width): the V^T projection [gw, M] takes 256 x 128
# workgroups at 512 x 8448 and 64 x 64 ones at 128 x 512.
@pytest.mark.parametrize("M,d,gw", [(8448, 2048, 512), (512, 512, 128)])
def test_projection_row_bias_whole_and_ragged_blocks(P, M, d, gw):
    """The transposed V projection (bias along rows) and the K projection
    (bias along columns, no residual) through whole and ragged wave blocks:
    the oracle's exact result on sampled tokens (integer lattice), M against
    M - 1 tokens on every shared element, canonical NaN."""
    rng = np.random.default_rng(97 + d)
    heads = d // 128
    x = lattice(rng, (M, d), -2, 2)
    w = {}
    for n in "qkvo":
        w["W" + n] = lattice(rng, (d, d), -2, 2)
        w["b" + n] = lattice(rng, (d,), -8, 8)
    x = with_specials(x, [5, M - 40, M - 2])
    g0 = d - gw  # the last head group's rows of Wk and Wv
    K1, V1 = attn_kv(P, x, w, heads, gw)
    K0, V0 = attn_kv(P, x[:M - 1], w, heads, gw)
    assert np.array_equal(K1[:M - 1], K0)
    assert np.array_equal(V1[:, :M - 1], V0)
    idx = np.unique(np.r_[0, 1, 5, 63, 64, M // 2, M - 65, M - 64, M - 40, M - 33, M - 2, M - 1])
    for got, name in ((K1[idx], "k"), (V1[:, idx].T, "v")):
        ref = oracle.linear(x[idx], w["W" + name][g0:], w["b" + name][g0:])
        assert np.array_equal(got, ref), name
    for got in (K1, V1):
        nan = np.isnan(f(got))
        assert nan.any() and np.all(got[nan] == 0x7FC0)
