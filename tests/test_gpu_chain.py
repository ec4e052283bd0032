"""The carried-chain GEMM kernel against the standard kernel, bit for bit.

A middle step of a K-split chain carries the fp32 accumulator in and out
([PSI] sec. II-B eq. (2): the down-projection's disjoint sum continued page by
page).  When the step has 1,024 input columns, whole 256 x 128 tiles, and an
even number of tiles for every CU, it runs on a kernel whose workgroups stay
resident and move the accumulator of one tile while the MFMAs of the next run.
A linear operator over column pages of 1,024 (first step, middle steps, last
step) is compared bitwise with the same operator over output-column pages,
where every tile takes the whole K on the standard kernel.  The token counts
give two, four and six tiles per workgroup on 256 CUs, a narrower output, a
single middle step, and a count the carried-chain kernel does not take
(ragged rows), which must agree as well.  One case is also checked against
the oracle on sampled rows.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import assert_bf16_close, dev, empty_bf16, host, make_arena

pytestmark = pytest.mark.gpu

KiB = 1024


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def linear(P, x, W, b, split, block):
    M, K = x.shape
    N = W.shape[0]
    m = P.pinned_matrix(W, b, split, block)
    pb = max(P.psi_matrix_page_bytes(m, p) for p in range(P.psi_matrix_pages(m)))
    acc = M * N * 4 if split == P.PSI_SPLIT_COLS else 0
    a = make_arena(2 * (pb + 64 * KiB) + acc + 4096, pb, 2)
    try:
        xd = dev(x)
        y = empty_bf16(M, N)
        P.psi_linear_paged(a, xd, M, K, m, None, y, 0)
        P.psi_arena_sync(a)
        return host(y)
    finally:
        P.psi_arena_destroy(a)
        torch.cuda.empty_cache()


@pytest.mark.parametrize("M,K,N", [(4096, 4096, 4096), (8192, 4096, 4096), (12288, 3072, 4096),
                                   (8192, 3072, 2048), (4000, 4096, 4096)])
def test_kernel_chain_same_bits_as_output_pages(P, M, K, N):
    rng = np.random.default_rng(M + K + N)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    W = synth.normal_bf16(rng, (N, K), 1.0 / np.sqrt(K))
    b = synth.normal_bf16(rng, (N,), 0.1)
    ref = linear(P, x, W, b, P.PSI_SPLIT_ROWS, 1024)
    got = linear(P, x, W, b, P.PSI_SPLIT_COLS, 1024)
    diff = np.flatnonzero(ref != got)
    assert diff.size == 0, f"{diff.size} outputs differ, first at {np.unravel_index(diff[0], ref.shape)}"
    if (M, K, N) == (8192, 4096, 4096):
        rows = np.sort(rng.choice(M, 12, replace=False))
        assert_bf16_close(got[rows], oracle.linear(x[rows], W, b), 2e-2)
