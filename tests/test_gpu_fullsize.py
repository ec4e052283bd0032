"""Parity at the full workload sizes, on sampled outputs the oracle computes
one by one, in the launch configuration the benchmark times (80 MiB arena,
8 MiB pages, 8-head groups, 1,024-channel FFN tiles, the O-projection over
output tiles with seven or eight pages), and in the paper's layout (two
pages + 8 MiB workspace, K-split O-projection).

Rows of an FFN are independent, so sampled rows of x go through the
oracle directly.  Attention rows depend on every key; the paged operator's
stage probes journal each head group's output O_g, so the oracle checks
(a) one head of every head-group page (heads 0, 9, 18, 31 of the 8-head
groups) on the sampled query rows against its own projections of that head
over all keys, and (b) the output projection + residual on the GPU's O
(identical inputs, as the paper's same-input probes do, [PSI] sec. IV-B).
The sampled rows hit every 256-row tile of the GEMM and attention
workgroups (one random row per tile, plus the first and the last row).

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import MiB, assert_bf16_close, dev, host, make_arena, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def sample_rows(M, n=None, seed=0, tile=256):
    """One random row in every `tile`-row block of [0, M), plus rows 0 and
    M - 1 (n is ignored: kept for call sites that name a count)."""
    rng = np.random.default_rng(seed)
    rows = {int(t + rng.integers(0, min(tile, M - t))) for t in range(0, M, tile)} | {0, M - 1}
    return np.array(sorted(rows))


# one head of each of the four 8-head groups
CHECK_HEADS = (0, 9, 18, 31)


def read_probe(P, j, role, branch, M, cols, step=0, block=0):
    out = np.empty((M, cols), np.uint16)
    P.psi_journal_read(j, P.key(step, block, branch, role), out, out.nbytes)
    return out


def check_attention(P, j, x_in, y, w, heads, gw, rows, ctx=None, step=0, otiles=False):
    """(a) one head of every head group on the sampled rows against the
    oracle's own projections of that head (its Q on those rows, its K and V
    over every key); (b) output projection + residual on the journaled O
    (per head group for the K-split, all groups at once for output tiles)."""
    M, d = x_in.shape
    if otiles:
        O = read_probe(P, j, P.PSI_ROLE_ATTN_O, -1, M, d, step)
    else:
        O = np.concatenate([read_probe(P, j, P.PSI_ROLE_ATTN_O, g, M, gw, step) for g in range(d // gw)],
                           axis=1)
    src = x_in if ctx is None else ctx
    xr = np.ascontiguousarray(x_in[rows])
    groups = set()
    for h in CHECK_HEADS:
        hs = slice(h * 128, (h + 1) * 128)
        groups.add(h * 128 // gw)
        Kh = oracle.linear(src, np.ascontiguousarray(w["Wk"][hs]), w["bk"][hs].copy())
        Vh = oracle.linear(src, np.ascontiguousarray(w["Wv"][hs]), w["bv"][hs].copy())
        Qh = oracle.linear(xr, np.ascontiguousarray(w["Wq"][hs]), w["bq"][hs].copy())
        Oh = oracle.attention(Qh, Kh, Vh, 1, 128)
        assert_bf16_close(O[rows][:, hs], Oh, what=f"attention head {h}")
    assert groups == set(range(d // gw)), "every head-group page is checked"
    ref = oracle.residual(x_in[rows], oracle.linear(np.ascontiguousarray(O[rows]), w["Wo"], w["bo"]))
    assert_bf16_close(y[rows], ref, what="output projection + residual")


@pytest.mark.parametrize("layout", ["tiles", "ksplit"])
def test_fullsize_block_8192_tokens(P, layout):
    """One block of the 8-block stack at full size (8,192 tokens, d 4,096,
    32 heads, FFN 16,384) in an 80 MiB arena of 8 MiB pages: the benchmark's
    seven pages with output-tile O-projection, or the paper's two pages +
    workspace with the K-split."""
    M, d, heads, hid = 8192, 4096, 32, 16384
    otiles = layout == "tiles"
    w = synth.block_weights(0, 0, d, hid)
    x0 = synth.stack_input(0, M, d)
    bw = P.block_weights(w, 1024, 1024, attn_out_tile=1024 if otiles else 0)
    ar = make_arena(80 * MiB, 8 * MiB, 7, 0) if otiles else make_arena(80 * MiB, 8 * MiB, 2, 8 * MiB)
    j = P.psi_journal_create(8 * MiB, 2, (4 + 16) * M * 1024 * 2 + MiB, 0)
    try:
        P.psi_arena_set_probe(ar, j, 0, 0)
        x = dev(x0)
        xt = torch.empty_like(x)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        P.psi_block_paged(ar, x, xt, M, heads, 128, bw, 1, acc, j, 0)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        y_attn, y = host(xt), host(x)
        rows = sample_rows(M)
        check_attention(P, j, x0, y_attn, w, heads, 1024, rows, otiles=otiles)
        # FFN on the GPU's own attention output (identical inputs), and its
        # first hidden tile from the stage probe
        xr = np.ascontiguousarray(y_attn[rows])
        assert_bf16_close(y[rows], oracle.ffn(xr, w["U"], w["a"], w["V"], w["b"], residual=True),
                          what="FFN sub-block")
        H0 = read_probe(P, j, P.PSI_ROLE_FFN_H, 0, M, 1024)
        pre = oracle.linear(xr, np.ascontiguousarray(w["U"][:1024]), w["a"][:1024].copy())
        assert_bf16_close(H0[rows], oracle.gelu_bf16(pre), what="hidden tile 0")
    finally:
        P.psi_arena_set_probe(ar, None)
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("layout", ["tiles", "ksplit"])
def test_fullsize_attention_self_and_cross(P, layout):
    """Attention sub-blocks at full size: 6,144 tokens self-attention, then
    cross-attention to 1,024 conditioning tokens, 32 heads of 128, 8-head
    groups, 80 MiB arena (eight pages with output tiles, as benchmarked; or
    two pages + workspace with the K-split)."""
    M, Mc, d, heads = 6144, 1024, 4096, 32
    otiles = layout == "tiles"
    c = synth.attn_case(0, M, Mc, d, cross=True)
    ar = make_arena(80 * MiB, 8 * MiB, 8, 0) if otiles else make_arena(80 * MiB, 8 * MiB, 2, 8 * MiB)
    j = P.psi_journal_create(8 * MiB, 2, 2 * 4 * M * 1024 * 2 + MiB, 0)
    try:
        x = dev(c["x"])
        ctx = dev(c["ctx"])
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        mats = {}
        for part in ("self", "cross"):
            w = c[part]
            mats[part] = [P.pinned_matrix(w["W" + n], w["b" + n], P.PSI_SPLIT_ROWS, 1024) for n in "qkv"] + \
                         [P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_ROWS if otiles else P.PSI_SPLIT_COLS,
                                          1024)]
        P.psi_arena_set_probe(ar, j, 0, 0)
        y1 = torch.empty_like(x)
        P.psi_attn_paged(ar, x, M, None, 0, heads, 128, *mats["self"], acc, y1, P.PSI_OP_RESIDUAL)
        P.psi_arena_set_probe(ar, j, 1, 0)
        y2 = torch.empty_like(x)
        P.psi_attn_paged(ar, y1, M, ctx, Mc, heads, 128, *mats["cross"], acc, y2, P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        P.psi_journal_sync(j)
        rows = sample_rows(M, seed=1)
        y1h, y2h = host(y1), host(y2)
        check_attention(P, j, c["x"], y1h, c["self"], heads, 1024, rows, step=0, otiles=otiles)
        check_attention(P, j, y1h, y2h, c["cross"], heads, 1024, rows, ctx=c["ctx"], step=1, otiles=otiles)
    finally:
        P.psi_arena_set_probe(ar, None)
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("cfg", ["d2048", "d4096"])
def test_fullsize_ffn(P, cfg):
    """FFN at d 2,048 / 8,192 hidden / 1,024 tokens in a 32 MiB arena with the
    fp32 accumulator in the arena, and at d 4,096 / 16,384 / 4,096 tokens in
    4 token chunks in an 80 MiB arena, on sampled rows."""
    if cfg == "d2048":
        M, d, hid, tile, chunks, arena, ws, ext = 1024, 2048, 8192, 2048, 1, 32, 0, False
    else:
        M, d, hid, tile, chunks, arena, ws, ext = 4096, 4096, 16384, 1024, 4, 80, 8, True
    c = synth.ffn_case(0, M, d, hid)
    U = P.pinned_matrix(c["U"], c["a"], P.PSI_SPLIT_ROWS, tile)
    V = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_COLS, tile)
    ar = make_arena(arena * MiB, 8 * MiB, 2, ws * MiB)
    try:
        x = dev(c["x"])
        y = torch.empty_like(x)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda") if ext else None
        P.psi_ffn_paged(ar, x, M, d, U, V, chunks, acc, y, 0)
        P.psi_arena_sync(ar)
        s = P.psi_arena_stats(ar)
        assert s.page_copies == 2 * hid // tile  # every page streamed exactly once
        rows = sample_rows(M, seed=2)
        yr = oracle.ffn(np.ascontiguousarray(c["x"][rows]), c["U"], c["a"], c["V"], c["b"])
        assert_bf16_close(host(y)[rows], yr, what=f"FFN {cfg}")
    finally:
        P.psi_arena_destroy(ar)


def test_fullsize_ffn_token_chunks_16384_tokens(P):
    """Page reuse across token chunks at twice the stack's token count: the
    FFN of 16,384 tokens (d 4,096, hidden 16,384, 1,024-channel tiles) in the
    benchmark's arena (80 MiB, seven 8 MiB pages, no workspace, fp32
    accumulator as declared live state) is refused in one chunk (its 32 MiB
    hidden tile exceeds the scratch) and runs in two, each page streamed
    once; sampled rows of every 256-row tile match the oracle.  At 8,192
    tokens, where one chunk fits, one and four chunks give the same bits."""
    d, hid = 4096, 16384
    c = synth.ffn_case(0, 16384, d, hid)
    U = P.pinned_matrix(c["U"], c["a"], P.PSI_SPLIT_ROWS, 1024)
    V = P.pinned_matrix(c["V"], c["b"], P.PSI_SPLIT_COLS, 1024)
    ar = make_arena(80 * MiB, 8 * MiB, 7, 0)
    try:
        M = 16384
        x = dev(c["x"])
        y = torch.empty_like(x)
        acc = torch.empty(M, d, dtype=torch.float32, device="cuda")
        with pytest.raises(P.PsiError) as e:
            P.psi_ffn_paged(ar, x, M, d, U, V, 1, acc, y, P.PSI_OP_RESIDUAL)
        assert e.value.status == P.PSI_E_SCRATCH_EXHAUSTED
        P.psi_arena_reset_stats(ar)
        P.psi_ffn_paged(ar, x, M, d, U, V, 2, acc, y, P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        s = P.psi_arena_stats(ar)
        assert s.page_copies == 2 * hid // 1024
        assert s.scratch_high_water == 8192 * 1024 * 2
        rows = sample_rows(M, seed=3)
        yr = oracle.ffn(np.ascontiguousarray(c["x"][rows]), c["U"], c["a"], c["V"], c["b"], residual=True)
        assert_bf16_close(host(y)[rows], yr, what="FFN 16,384 tokens in two chunks")
        half = 8192
        outs = []
        for ch in (1, 4):
            y2 = torch.empty(half, d, dtype=torch.int16, device="cuda")
            P.psi_ffn_paged(ar, x[:half], half, d, U, V, ch, acc[:half], y2, P.PSI_OP_RESIDUAL)
            P.psi_arena_sync(ar)
            outs.append(host(y2))
        assert np.array_equal(outs[0], outs[1])
        assert np.array_equal(outs[0], host(y)[:half])  # rows do not depend on the other rows
    finally:
        P.psi_arena_destroy(ar)
