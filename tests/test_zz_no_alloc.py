"""The allocation-free projection against psi_linear_paged on the same
resident matrix: bitwise equal outputs on two calls in a row (the second
smaller, so it finds the first call's accumulator in the static array), for
the K-split and output-column splits, with and without the residual; the
oracle bounds both; oversized accumulators are refused before any launch.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import MiB, assert_bf16_close, dev, empty_bf16, host, make_arena, stream_handle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def paged_reference(P, x, M, K, Wr, flags):
    """psi_linear_paged on the resident matrix, accumulator in arena scratch."""
    N = Wr.rows
    ar = make_arena(4 * MiB + M * N * 4, 1 * MiB, 2)
    try:
        y = empty_bf16(M, N)
        P.psi_linear_paged(ar, x, M, K, Wr, None, y, flags)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("split,block,resid", [("cols", 256, False), ("cols", 200, True),
                                               ("rows", 128, False), ("rows", 96, True)])
def test_noalloc_linear_matches_paged(P, split, block, resid):
    K = N = 1024
    c = synth.linear_case(seed=41, M=640, K=K, N=N)
    sp = P.PSI_SPLIT_COLS if split == "cols" else P.PSI_SPLIT_ROWS
    Wr = P.resident_matrix(P.pinned_matrix(c["W"], c["b"], sp, block))
    flags = P.PSI_OP_RESIDUAL if resid else 0
    xd = dev(c["x"])
    for M in (640, 200):  # second call smaller: the static array holds the first call's values
        x = xd[:M]
        y = empty_bf16(M, N)
        P.psi_linear_resident_noalloc(x, M, K, Wr, y, flags, stream_handle())
        got = host(y)
        ref = paged_reference(P, x, M, K, Wr, flags)
        assert np.array_equal(got, ref), (split, block, resid, M)
        yr = oracle.linear(np.ascontiguousarray(c["x"][:M]), c["W"], c["b"])
        if resid:
            yr = oracle.residual(np.ascontiguousarray(c["x"][:M]), yr)
        assert_bf16_close(got, yr)


def test_noalloc_linear_refusals(P):
    c = synth.linear_case(seed=42, M=64, K=256, N=512)
    W = P.pinned_matrix(c["W"], c["b"], P.PSI_SPLIT_COLS, 128)
    Wr = P.resident_matrix(W)
    x = dev(c["x"])
    y = empty_bf16(64, 512)
    before = host(y).copy()
    big = P.PSI_NOALLOC_SCRATCH_BYTES // (512 * 4) + 1  # rows whose accumulator exceeds the array
    with pytest.raises(P.PsiError) as e:
        P.psi_linear_resident_noalloc(x, big, 256, Wr, y, 0, stream_handle())
    assert e.value.status == P.PSI_E_SCRATCH_EXHAUSTED
    with pytest.raises(P.PsiError) as e:  # streamed (pinned host) weights are refused
        P.psi_linear_resident_noalloc(x, 64, 256, W, y, 0, stream_handle())
    assert e.value.status == P.PSI_E_INVALID
    with pytest.raises(P.PsiError) as e:
        P.psi_linear_resident_noalloc(x, 64, 256, Wr, y, P.PSI_OP_STORE_ACC, stream_handle())
    assert e.value.status == P.PSI_E_INVALID
    torch.cuda.synchronize()
    assert np.array_equal(host(y), before)  # nothing was launched
