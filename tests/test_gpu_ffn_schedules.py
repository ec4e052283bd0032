"""FFN schedules over output tiles of the down-projection ([PSI] sec. III-B
"FFN reuse" and the recompute scheduling baseline) on the GPU.

The paper computes each hidden tile once, journals it and reloads it for
every down-projection output tile, and compares that with recomputing it;
both keep the ordered down-projection accumulation, so the outputs do not
change (its Table IV: unchanged BF16 outputs).  Here both schedules are
checked bitwise against the resident K-split schedule (psi_ffn_paged) and
against the oracle, on ragged token counts, ragged output tiles and
ragged hidden tiles, and the journal traffic is checked against the
schedule: one D2H of every hidden tile, one H2D per (output tile, hidden
tile).

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import MiB, assert_bf16_close, dev, empty_bf16, host, make_arena

pytestmark = pytest.mark.gpu

KiB = 1024


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def run_resident(P, c, tile, residual=False):
    """psi_ffn_paged: H_J resident, K-split pages V[:, J]."""
    x = c["x"]
    M, d = x.shape
    U = P.pinned_matrix(c["U"], c["a"], P.PSI_SPLIT_ROWS, tile)
    V = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_COLS, tile)
    ar = make_arena(8 * MiB, 512 * KiB, 3)
    try:
        xd = dev(x)
        y = xd if residual else empty_bf16(M, d)
        P.psi_ffn_paged(ar, xd, M, d, U, V, 1, None, y, P.PSI_OP_RESIDUAL if residual else 0)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


def run_tiled(P, c, th, to, schedule, residual=False, n_pages=3):
    """psi_ffn_tiled with hidden tile th and output tile to; returns the
    output and the journal counters (D2H bytes, H2D bytes, entries)."""
    x = c["x"]
    M, d = x.shape
    h = c["U"].shape[0]
    U = P.pinned_matrix(c["U"], c["a"], P.PSI_SPLIT_ROWS, th)
    Vo = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_ROWS, to)
    ar = make_arena(8 * MiB, 512 * KiB, n_pages)
    j = P.psi_journal_create(1 * MiB, 2, h * M * 2 + MiB)
    try:
        xd = dev(x)
        y = xd if residual else empty_bf16(M, d)
        P.psi_ffn_tiled(ar, xd, M, d, U, Vo, schedule, j, 3, 1, y, P.PSI_OP_RESIDUAL if residual else 0)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        return host(y), P.psi_journal_counters(j)
    finally:
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("M,th,to", [(200, 256, 96), (64, 128, 256), (130, 384, 80)])
def test_ffn_reuse_and_recompute_match_resident_bitwise(P, M, th, to):
    """Both output-tile schedules reproduce the resident K-split FFN bit for
    bit (same hidden tiles, same order per output) and match the oracle."""
    c = synth.ffn_case(seed=7, M=M, d=256, hidden=1024)
    ref = run_resident(P, c, th)
    assert_bf16_close(ref, oracle.ffn(c["x"], c["U"], c["a"], c["V"], c["b"]), what="resident FFN")
    for sched in (P.PSI_FFN_REUSE, P.PSI_FFN_RECOMPUTE):
        got, _ = run_tiled(P, c, th, to, sched)
        assert np.array_equal(got, ref), f"schedule {sched}, M {M}, t_h {th}, t_o {to}"


def test_ffn_reuse_journal_traffic(P):
    """FFN reuse moves every hidden tile to the host once and back once per
    output tile; the recompute baseline uses no journal."""
    M, d, h, th, to = 96, 256, 1024, 256, 64
    c = synth.ffn_case(seed=8, M=M, d=d, hidden=h)
    _, (d2h, h2d, entries) = run_tiled(P, c, th, to, P.PSI_FFN_REUSE)
    assert entries == h // th
    assert d2h == h * M * 2
    assert h2d == (d // to) * h * M * 2
    _, (d2h, h2d, entries) = run_tiled(P, c, th, to, P.PSI_FFN_RECOMPUTE)
    assert (d2h, h2d, entries) == (0, 0, 0)


def test_ffn_schedules_residual_in_place_and_two_pages(P):
    """With a single output tile y may alias x (residual write); the
    recompute schedule also runs in a two-slot arena (one slot holds the
    output tile, the other streams U)."""
    c = synth.ffn_case(seed=9, M=72, d=128, hidden=512)
    ref = run_resident(P, c, 128, residual=True)
    assert_bf16_close(ref, oracle.ffn(c["x"], c["U"], c["a"], c["V"], c["b"], residual=True))
    for sched in (P.PSI_FFN_REUSE, P.PSI_FFN_RECOMPUTE):
        got, _ = run_tiled(P, c, 128, 128, sched, residual=True, n_pages=2)
        assert np.array_equal(got, ref), sched
