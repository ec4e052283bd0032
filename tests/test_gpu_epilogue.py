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
FFN (GELU epilogue, then the carried down-projection with residual), for the
256 x 128 and the 64 x 64 tile shapes.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

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
