"""Low-live-state mode on the GPU ([PSI] sec. III-B: intermediate state is
retained on device or stored in the host journal for later use).

* psi_attn_tiled keeps the head-group outputs O_g in the journal and runs
  the O-projection over output tiles; each output element still sums the
  same channels in the same order, so it reproduces psi_attn_paged bit for
  bit (self- and cross-attention, ragged output tiles, y aliasing x);
* the FFN reuse schedule now double-buffers its hidden tiles and may write
  its output over its input;
* psi_block_lowlive (x the only device state) reproduces psi_block_paged
  bit for bit over a stack of blocks that share one journal, whose store
  holds a single block's intermediates (psi_journal_reset reuses it in
  stream order), in both journal transports.

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


def attn_mats(P, w, gw, to=0):
    ms = [P.pinned_matrix(w["W" + n], w["b" + n], P.PSI_SPLIT_ROWS, gw) for n in "qkv"]
    ms.append(P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_ROWS, to) if to else
              P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_COLS, gw))
    return ms


def run_attn(P, x, w, heads, dh, gw, *, to=0, ctx=None, flags=0, inplace=False):
    M, d = x.shape
    Mc = 0 if ctx is None else ctx.shape[0]
    ar = make_arena(16 * MiB, max(gw, to or 0) * d * 2, 2)
    j = P.psi_journal_create(MiB, 2, M * d * 2 + MiB) if to else None
    try:
        xd = dev(x)
        cd = dev(ctx) if ctx is not None else None
        y = xd if inplace else empty_bf16(M, d)
        fl = flags | P.PSI_OP_RESIDUAL
        if to:
            P.psi_attn_tiled(ar, xd, M, cd, Mc, heads, dh, *attn_mats(P, w, gw, to), j, 0, 0, y, fl)
        else:
            P.psi_attn_paged(ar, xd, M, cd, Mc, heads, dh, *attn_mats(P, w, gw), None, y, fl)
        P.psi_arena_sync(ar)
        out = host(y)
        counters = None
        if j:
            P.psi_journal_sync(j)
            counters = P.psi_journal_counters(j)
        return out, counters
    finally:
        if j:
            P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("dh,gw,to,cross", [(128, 256, 128, False), (128, 128, 96, True),
                                            (64, 192, 512, False)])
def test_attn_tiled_matches_paged_bitwise(P, dh, gw, to, cross):
    """O-projection over output tiles from journaled head-group outputs
    gives psi_attn_paged's bits (ragged output tiles: 96 of 512; ragged
    head groups: 192 of 512 with 64-dim heads); the journal moves every O_g
    to the host once and back once per output tile."""
    rng = np.random.default_rng(40 + dh + gw)
    d, M = 512, 150
    heads = d // dh
    x = synth.normal_bf16(rng, (M, d), 1.0)
    ctx = synth.normal_bf16(rng, (77, d), 1.0) if cross else None
    w = synth.attn_weights(rng, d)
    ref, _ = run_attn(P, x, w, heads, dh, gw, ctx=ctx)
    got, (d2h, h2d, entries) = run_attn(P, x, w, heads, dh, gw, to=to, ctx=ctx)
    assert np.array_equal(got, ref)
    n_g, n_o = -(-d // gw), -(-d // to)
    assert entries == n_g and d2h == M * d * 2 and h2d == n_o * M * d * 2
    assert_bf16_close(got, oracle.attn_sublayer(x, w["Wq"], w["bq"], w["Wk"], w["bk"], w["Wv"], w["bv"],
                                                w["Wo"], w["bo"], heads, dh, ctx=ctx))


def test_attn_tiled_in_place_and_bf16_numerator(P):
    """y may alias x; the numerator options give the paged operator's bits."""
    rng = np.random.default_rng(45)
    d, M, heads = 256, 130, 2
    x = synth.normal_bf16(rng, (M, d), 1.0)
    w = synth.attn_weights(rng, d)
    for fl in (0, P.PSI_OP_BF16_SOFTMAX, P.PSI_OP_ATTN_P2):
        ref, _ = run_attn(P, x, w, heads, 128, 128, flags=fl)
        got, _ = run_attn(P, x, w, heads, 128, 128, to=64, flags=fl, inplace=True)
        assert np.array_equal(got, ref), fl


def test_ffn_reuse_in_place_many_output_tiles(P):
    """The FFN reuse schedule writes its output over its input even with
    several output tiles (all hidden tiles are computed first)."""
    c = synth.ffn_case(seed=46, M=96, d=256, hidden=768)
    x = c["x"]
    M, d = x.shape
    U = P.pinned_matrix(c["U"], c["a"], P.PSI_SPLIT_ROWS, 256)
    V = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_COLS, 256)
    Vo = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_ROWS, 64)
    ar = make_arena(8 * MiB, 512 * KiB, 2)
    j = P.psi_journal_create(MiB, 2, 768 * M * 2 + MiB)
    try:
        xd = dev(x)
        y = empty_bf16(M, d)
        P.psi_ffn_paged(ar, xd, M, d, U, V, 1, None, y, P.PSI_OP_RESIDUAL)
        P.psi_ffn_tiled(ar, xd, M, d, U, Vo, P.PSI_FFN_REUSE, j, 0, 0, xd, P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        assert np.array_equal(host(xd), host(y))
    finally:
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("ring", [False, True])
def test_lowlive_stack_matches_paged_stack_bitwise(P, ring):
    """Three blocks in low-live-state mode (only x on the device, one
    journal whose store holds one block's intermediates) give the bits of
    three psi_block_paged blocks."""
    M, d, heads, h, gw = 160, 256, 2, 1024, 128
    x0 = synth.stack_input(47, M, d)
    ws = [synth.block_weights(47, i, d, h) for i in range(3)]
    ar = make_arena(16 * MiB, 512 * KiB, 2)
    flags = P.PSI_JOURNAL_RING if ring else 0
    store = M * (d + h) * 2 + 64 * KiB
    j = P.psi_journal_create(128 * KiB, 4, store, flags)
    try:
        xr = dev(x0)
        xt = torch.empty_like(xr)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        for w in ws:
            P.psi_block_paged(ar, xr, xt, M, heads, 128, P.block_weights(w, gw, 256), 1, acc, None, 0)
        xl = dev(x0)
        for w in ws:
            bw = P.block_weights(w, gw, 256, attn_out_tile=64, ffn_out_tile=128)
            P.psi_block_lowlive(ar, xl, M, heads, 128, bw, j, 0)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        assert np.array_equal(host(xl), host(xr))
        d2h, h2d, entries = P.psi_journal_counters(j)
        assert entries == d // gw + h // 256          # the last block's entries
        assert d2h == 3 * M * (d + h) * 2
        assert h2d == 3 * M * 2 * ((d // 64) * d + (d // 128) * h)
    finally:
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


def test_lowlive_block_ragged_medium_size_matches_paged(P):
    """One low-live block at a size spanning many tiles with ragged token
    count, output tiles and hidden tiles (777 tokens, d 1,024, 8 heads of
    128, FFN 4,096 in 768-channel tiles; attention output tiles of 384, FFN
    output tiles of 320) gives psi_block_paged's bits and is within the
    tolerance of the oracle's block."""
    M, d, heads, h, gw = 777, 1024, 8, 4096, 256
    x0 = synth.stack_input(48, M, d)
    w = synth.block_weights(48, 0, d, h)
    ar = make_arena(32 * MiB, 4 * MiB, 3)
    j = P.psi_journal_create(MiB, 2, M * (d + h) * 2 + MiB)
    try:
        xr = dev(x0)
        xt = torch.empty_like(xr)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        P.psi_block_paged(ar, xr, xt, M, heads, 128, P.block_weights(w, gw, 768), 1, acc, None, 0)
        xl = dev(x0)
        P.psi_block_lowlive(ar, xl, M, heads, 128, P.block_weights(w, gw, 768, attn_out_tile=384,
                                                                    ffn_out_tile=320), j, 0)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        got = host(xl)
        assert np.array_equal(got, host(xr))
        assert_bf16_close(got, oracle.block(x0, w, heads, 128))
    finally:
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("recompute", [False, True])
def test_two_d_page_tiles_bitwise(P, recompute):
    """2-D page tiles (PSI_SPLIT_TILES): wide output tiles cut into pages of
    whole hidden tiles / head groups, with ragged row tiles, ragged column
    pages and a ragged last hidden tile, give the bits of the row-split
    output tiles and of psi_block_paged, and reload each journaled hidden
    state once per row tile (777 tokens, d 1,024, FFN 3,960 in 800-channel
    tiles, the last 760: V in 320 x 2,400 pages, Wo in 384 x 512 pages)."""
    M, d, heads, h, gw, th = 777, 1024, 8, 3960, 256, 800
    x0 = synth.stack_input(49, M, d)
    w = synth.block_weights(49, 0, d, h)
    ar = make_arena(32 * MiB, 4 * MiB, 3)
    j = P.psi_journal_create(MiB, 2, M * (d + h) * 2 + MiB)
    try:
        xr = dev(x0)
        xt = torch.empty_like(xr)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        P.psi_block_paged(ar, xr, xt, M, heads, 128, P.block_weights(w, gw, th), 1, acc, None, 0)
        ref = host(xr)
        # the FFN alone, row-split against 2-D tiles, on the same input
        U = P.pinned_matrix(w["U"], w["a"], P.PSI_SPLIT_ROWS, th)
        Vr = P.pinned_matrix(w["V"], w["b"], P.PSI_SPLIT_ROWS, 320)
        Vt = P.pinned_matrix(w["V"], w["b"], P.PSI_SPLIT_TILES, 320, 2400)
        assert P.psi_matrix_pages(Vt) == 4 * 2
        sched = P.PSI_FFN_RECOMPUTE if recompute else P.PSI_FFN_REUSE
        outs, reloads = [], []
        for V in (Vr, Vt):
            P.psi_journal_reset(j)
            P.psi_journal_sync(j)
            _, h2d0, _ = P.psi_journal_counters(j)
            y = empty_bf16(M, d)
            P.psi_ffn_tiled(ar, dev(x0), M, d, U, V, sched, j, 0, 1, y, P.PSI_OP_RESIDUAL)
            P.psi_arena_sync(ar)
            P.psi_journal_sync(j)
            outs.append(host(y))
            reloads.append(P.psi_journal_counters(j)[1] - h2d0)
        assert np.array_equal(outs[0], outs[1])
        if not recompute:
            assert reloads == [4 * M * h * 2, 4 * M * h * 2]  # one reload per row tile (4 either way)
        if recompute:
            return
        # the whole low-live block with 2-D tiles in both output-tile schedules
        xl = dev(x0)
        bw = P.block_weights(w, gw, th, attn_out_tile=384, ffn_out_tile=1024, attn_out_cols=512,
                             ffn_out_cols=1600)
        P.psi_journal_reset(j)
        P.psi_journal_sync(j)
        _, h2d0, _ = P.psi_journal_counters(j)
        P.psi_block_lowlive(ar, xl, M, heads, 128, bw, j, 0)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        assert np.array_equal(host(xl), ref)
        _, h2d1, _ = P.psi_journal_counters(j)
        assert h2d1 - h2d0 == 3 * M * d * 2 + 1 * M * h * 2  # 3 attention row tiles, 1 FFN row tile
    finally:
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)
