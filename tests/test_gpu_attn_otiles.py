"""Attention O-projection over output tiles on the GPU.

With Wo split by rows, psi_attn_paged (and psi_attn_paged_ext) keep every
head group's output O_g in one [M, d] BF16 buffer (acc_dev's memory, or
scratch) and run the O-projection once per output tile over the full K:
each output sums the same products in the same order as the K-split over
head groups with its carried fp32 accumulator ([PSI] sec. II-B: the
disjoint partition preserves the dense summation), so the two layouts
give the same bits.  Ragged output tiles, cross-attention, y aliasing x,
the numerics options, the extended attention and a stack of blocks are
covered; one case is also checked against the oracle.

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


def mats(P, w, gw, to=0):
    ms = [P.pinned_matrix(w["W" + n], w["b" + n], P.PSI_SPLIT_ROWS, gw) for n in "qkv"]
    ms.append(P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_ROWS, to) if to else
              P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_COLS, gw))
    return ms


def run(P, x, w, heads, dh, gw, *, to=0, ctx=None, flags=0, inplace=False, use_acc=True, nr=None):
    M, d = x.shape
    Mc = 0 if ctx is None else ctx.shape[0]
    ar = make_arena(24 * MiB, max(gw, to or 0) * d * 2, 3)
    try:
        xd = dev(x)
        cd = dev(ctx) if ctx is not None else None
        y = xd if inplace else empty_bf16(M, d)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda") if use_acc else None
        fl = flags | P.PSI_OP_RESIDUAL
        if nr is None:
            P.psi_attn_paged(ar, xd, M, cd, Mc, heads, dh, *mats(P, w, gw, to), acc, y, fl)
        else:
            P.psi_attn_paged_ext(ar, xd, M, cd, Mc, heads, dh, *mats(P, w, gw, to), nr, acc, y, fl)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("dh,gw,to,cross,use_acc", [(128, 256, 256, False, True), (128, 128, 96, True, True),
                                                    (64, 192, 320, False, False), (128, 256, 512, True, False)])
def test_output_tiles_match_ksplit_bitwise(P, dh, gw, to, cross, use_acc):
    """Output tiles of 256 (= the group), 96 (ragged, narrower than a
    group), 320 and 512 give the K-split's bits, with the head-group outputs
    in acc_dev's memory or in scratch; ragged head groups (192 of 512)."""
    rng = np.random.default_rng(70 + gw + to)
    d, M = 512, 150
    heads = d // dh
    x = synth.normal_bf16(rng, (M, d), 1.0)
    ctx = synth.normal_bf16(rng, (77, d), 1.0) if cross else None
    w = synth.attn_weights(rng, d)
    ref = run(P, x, w, heads, dh, gw, ctx=ctx)
    got = run(P, x, w, heads, dh, gw, to=to, ctx=ctx, use_acc=use_acc)
    assert np.array_equal(got, ref)
    if to == 96:
        assert_bf16_close(got, oracle.attn_sublayer(x, w["Wq"], w["bq"], w["Wk"], w["bk"], w["Wv"], w["bv"],
                                                    w["Wo"], w["bo"], heads, dh, ctx=ctx))


def test_output_tiles_in_place_and_numerics_options(P):
    """y may alias x (each tile reads the residual of its own columns only);
    baseline bias, BF16 numerator and two-term weights keep the K-split's
    bits too."""
    rng = np.random.default_rng(75)
    d, M, heads = 256, 130, 2
    x = synth.normal_bf16(rng, (M, d), 1.0)
    w = synth.attn_weights(rng, d)
    for fl in (0, P.PSI_OP_BASELINE_BIAS, P.PSI_OP_BF16_SOFTMAX, P.PSI_OP_ATTN_P2):
        ref = run(P, x, w, heads, 128, 128, flags=fl)
        got = run(P, x, w, heads, 128, 128, to=64, flags=fl, inplace=True)
        assert np.array_equal(got, ref), fl


def test_extended_attention_output_tiles(P):
    """psi_attn_paged_ext (Q/K RMS normalisation and RoPE, 64-dim heads)
    with output tiles gives its K-split bits; the O tiles read the full-width
    Q buffer that the attention overwrote with O."""
    c = synth.attn_ext_case(seed=76, M=126, d=512)
    M, d = c["x"].shape
    cq, sq = synth.rope_tables(M, 64)
    g = [torch.from_numpy(c[k].view(np.int16)).pin_memory() for k in ("gq", "gk")]
    ct, st = torch.from_numpy(cq).cuda(), torch.from_numpy(sq).cuda()
    nr = P.qk_norm_rope(g[0], g[1], 1e-6, 0, ct, st)
    ref = run(P, c["x"], c["w"], 8, 64, 128, nr=nr)
    for to, use_acc in ((128, True), (192, False)):
        got = run(P, c["x"], c["w"], 8, 64, 128, to=to, nr=nr, use_acc=use_acc)
        assert np.array_equal(got, ref), to


def test_block_stack_output_tiles_match_ksplit(P):
    """Two psi_block_paged blocks with Wo split into output tiles of 128
    give the K-split stack's bits (the fp32 accumulator buffer holds the
    head-group outputs during attention, then the FFN's accumulator)."""
    M, d, heads, h, gw = 200, 256, 2, 1024, 128
    x0 = synth.stack_input(77, M, d)
    ws = [synth.block_weights(77, i, d, h) for i in range(2)]
    outs = []
    for to in (0, 128):
        ar = make_arena(16 * MiB, 512 * KiB, 3)
        try:
            x = dev(x0)
            xt = torch.empty_like(x)
            acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
            for w in ws:
                P.psi_block_paged(ar, x, xt, M, heads, 128, P.block_weights(w, gw, 256, attn_out_tile=to), 2,
                                  acc, None, 0)
            P.psi_arena_sync(ar)
            outs.append(host(x))
        finally:
            P.psi_arena_destroy(ar)
    assert np.array_equal(outs[0], outs[1])


def test_lent_scratch_slots_keep_bits(P):
    """Operators lend their idle scratch as extra page slots.  Two blocks
    with output-tile attention (no arena scratch) and the FFN, with every
    copy and launch delayed by a pseudo-random 0-63 us (PSI_ARENA_JITTER),
    give the bits of the sync-copy transport control, which lends nothing;
    pages did go through lent slots."""
    M, d, heads, h, gw = 200, 256, 2, 1024, 128
    x0 = synth.stack_input(78, M, d)
    ws = [synth.block_weights(78, i, d, h) for i in range(2)]
    bws = [P.block_weights(w, gw, 256, attn_out_tile=128) for w in ws]
    outs, lent = [], []
    for flags in (P.PSI_ARENA_SYNC_COPY, P.PSI_ARENA_JITTER):
        ar = make_arena(4 * MiB, 128 * KiB, 3, flags=flags)
        try:
            x = dev(x0)
            xt = torch.empty_like(x)
            acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
            for bw in bws:
                P.psi_block_paged(ar, x, xt, M, heads, 128, bw, 1, acc, None, 0)
            P.psi_arena_sync(ar)
            outs.append(host(x))
            lent.append(P.psi_arena_stats(ar).lent_page_copies)
        finally:
            P.psi_arena_destroy(ar)
    assert np.array_equal(outs[0], outs[1])
    assert lent[0] == 0 and lent[1] > 0, lent
