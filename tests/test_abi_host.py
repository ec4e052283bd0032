"""Host-side tests of the C-ABI library (no GPU needed).

The library must load and export every entry point ``include/psi.h``
declares; the arena carve, the operator feasibility plans and the page
lifecycle are host logic and are checked here through a dry-run arena
(``PSI_ARENA_DRY_RUN``: no device memory, no HIP calls, no compute).

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import os
import re
import subprocess

import numpy as np
import pytest

from memory_bounded_weight_amd import psi
from tests import golden

MiB = 1 << 20
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "psi.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psi_[a-z_0-9]+)\s*\(", text)))


def test_exports_match_header():
    declared = header_functions()
    assert declared, "no declarations parsed"
    assert sorted(psi.EXPORTS) == declared
    out = subprocess.run(["nm", "-D", "--defined-only", psi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (psi_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert "gfx950" in psi.psi_version()


def test_library_has_gfx950_code_object():
    """The shared library embeds an offload bundle for gfx950."""
    blob = open(psi.LIB_PATH, "rb").read()
    assert b"__CLANG_OFFLOAD_BUNDLE__" in blob
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def desc(arena_mib, page_mib, n_pages=2, ws_mib=0, flags=psi.PSI_ARENA_DRY_RUN):
    return psi.arena_desc(int(arena_mib * MiB), int(page_mib * MiB), n_pages, int(ws_mib * MiB), 0,
                          None, flags)


# ------------------------------------------------------------------ carve

def test_arena_carve_paper_split():
    """[PSI] sec. IV-A / Fig. 1: 80 MiB = 8 + 8 pages + 8 workspace + 56
    state/scratch; here the two 64 KiB bias slots come out of the 56 MiB
    (they are the bounded metadata term of eq. (1))."""
    L = psi.psi_arena_plan(desc(80, 8, 2, 8))
    assert L.page_off[0] == 0 and L.page_off[1] == 8 * MiB
    assert L.bias_off[0] == 16 * MiB and L.bias_off[1] == 16 * MiB + 64 * 1024
    assert L.bias_slot_bytes == 64 * 1024
    assert L.workspace_off == 16 * MiB + 128 * 1024
    assert L.scratch_off == 24 * MiB + 128 * 1024
    assert L.scratch_bytes == 56 * MiB - 128 * 1024
    assert L.total_bytes == 80 * MiB


def test_arena_three_pages_same_footprint():
    """The 8 MiB workspace reassigned to a third page slot keeps the 80 MiB
    arena and the scratch size of the two-page carve."""
    L2 = psi.psi_arena_plan(desc(80, 8, 2, 8))
    L3 = psi.psi_arena_plan(desc(80, 8, 3, 0))
    assert L3.page_off[2] == 16 * MiB and L3.bias_off[0] == 24 * MiB
    assert L3.scratch_bytes == L2.scratch_bytes
    assert L3.total_bytes == 80 * MiB


def test_arena_too_small():
    with pytest.raises(psi.PsiError) as e:
        psi.psi_arena_plan(desc(16, 8, 2, 8))
    assert e.value.status == psi.PSI_E_ARENA_TOO_SMALL
    with pytest.raises(psi.PsiError) as e:
        psi.psi_arena_plan(desc(80, 8, 0))
    assert e.value.status == psi.PSI_E_INVALID


# ---------------------------------------------------- matrices and packing

def test_pack_matrix_column_pages():
    rng = np.random.default_rng(0)
    W = rng.integers(0, 65535, size=(6, 40), dtype=np.uint16)
    out = np.zeros(6 * 40, np.uint16)
    psi.psi_pack_matrix(W, 6, 40, psi.PSI_SPLIT_COLS, 16, out)
    pages = [W[:, 0:16], W[:, 16:32], W[:, 32:40]]
    assert np.array_equal(out, np.concatenate([p.ravel() for p in pages]))
    out2 = np.zeros(6 * 40, np.uint16)
    psi.psi_pack_matrix(W, 6, 40, psi.PSI_SPLIT_ROWS, 4, out2)
    assert np.array_equal(out2, W.ravel())
    m = psi.make_matrix(out, None, 6, 40, psi.PSI_SPLIT_COLS, 16)
    assert psi.psi_matrix_pages(m) == 3
    assert [psi.psi_matrix_page_bytes(m, p) for p in range(3)] == [6 * 16 * 2, 6 * 16 * 2, 6 * 8 * 2]


def fake_matrix(rows, cols, split, block, bias=True):
    # plans never dereference the image; any non-null address works
    return psi.make_matrix(0x1000, 0x2000 if bias else None, rows, cols, split, block)


def cfg5_attn(block_cols=1024):
    return [fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, block_cols) for _ in range(3)] + \
           [fake_matrix(4096, 4096, psi.PSI_SPLIT_COLS, block_cols)]


def cfg5_ffn(tile=1024):
    return (fake_matrix(16384, 4096, psi.PSI_SPLIT_ROWS, tile),
            fake_matrix(4096, 16384, psi.PSI_SPLIT_COLS, tile))


TABLE_V_OUTCOME = {"scratch_exhausted": psi.PSI_E_SCRATCH_EXHAUSTED, "complete": psi.PSI_OK,
                   "weight_tile_exceeds_page": psi.PSI_E_PAGE_TOO_SMALL}


@pytest.mark.parametrize("arena,page,expect", [(int(a), int(p), TABLE_V_OUTCOME[o])
                                               for a, p, o in golden.rows("table_v_capacity.txt")])
def test_capacity_outcomes_like_table_v(arena, page, expect):
    """[PSI] Table V (tests/golden) lists six arena/page capacities for one
    block with tiles held fixed: 48/8 and 64/8 exhaust scratch, 80/8, 96/8,
    96/16 complete, 80/4 fails because a weight tile exceeds the page.  With
    the stack's tiles (8-head groups, 1,024-channel FFN tiles, 8,192 tokens,
    8 MiB workspace) the same six settings give the same outcome pattern."""
    d = desc(arena, page, 2, 8, 0)
    Wq, Wk, Wv, Wo = cfg5_attn()
    st_a, need_a = psi.psi_attn_plan(d, 8192, 0, 32, 128, Wq, Wk, Wv, Wo, True)
    U, V = cfg5_ffn()
    st_f, need_f = psi.psi_ffn_plan(d, 8192, 4096, U, V, 1, True)
    worst = st_a if st_a != psi.PSI_OK else st_f
    assert worst == expect, (st_a, st_f, psi.psi_last_error())
    if expect == psi.PSI_OK:
        assert need_a == 3 * 8192 * 1024 * 2  # Q, K, V^T of one 8-head group
        assert need_f == 8192 * 1024 * 2      # one hidden tile for all tokens


def test_plan_errors_and_scratch_accumulator():
    d = desc(32, 8, 2, 0, 0)  # the FFN d=2048 configuration: 32 MiB arena, 8 MiB pages
    U = fake_matrix(8192, 2048, psi.PSI_SPLIT_ROWS, 2048)
    V = fake_matrix(2048, 8192, psi.PSI_SPLIT_COLS, 2048)
    st, need = psi.psi_ffn_plan(d, 1024, 2048, U, V, 1, False)  # fp32 ACC in the arena
    assert st == psi.PSI_OK and need == 1024 * 2048 * 2 + 1024 * 2048 * 4
    st, _ = psi.psi_ffn_plan(d, 1024, 2048, V, U, 1, False)
    assert st == psi.PSI_E_INVALID
    U2 = fake_matrix(8192, 2048, psi.PSI_SPLIT_ROWS, 4096)  # 16 MiB tile > 8 MiB page
    V2 = fake_matrix(2048, 8192, psi.PSI_SPLIT_COLS, 4096)
    st, _ = psi.psi_ffn_plan(d, 1024, 2048, U2, V2, 1, True)
    assert st == psi.PSI_E_PAGE_TOO_SMALL
    st, _ = psi.psi_ffn_plan(d, 4096, 2048, U, V, 1, False)  # ACC 32 MiB no longer fits
    assert st == psi.PSI_E_SCRATCH_EXHAUSTED
    Wq, Wk, Wv, Wo = cfg5_attn()
    st, _ = psi.psi_attn_plan(desc(80, 8, 2, 8, 0), 8192, 0, 32, 64, Wq, Wk, Wv, Wo, True)
    assert st == psi.PSI_E_INVALID  # head_dim 128 only
    Wk_bad = fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, 512)
    st, _ = psi.psi_attn_plan(desc(80, 8, 2, 8, 0), 8192, 0, 32, 128, Wq, Wk_bad, Wv, Wo, True)
    assert st == psi.PSI_E_INVALID
    odd = fake_matrix(64, 36, psi.PSI_SPLIT_ROWS, 16)
    st, _ = psi.psi_linear_plan(desc(1, 0.25, 2, 0, 0), 8, 36, odd, True)
    assert st == psi.PSI_E_ALIGN


# ------------------------------------------------------- page lifecycle

def test_page_lifecycle_dry_run():
    """[PSI] sec. II-A rule 2 and sec. II-D: at most one unreleased request
    per page; free -> filling -> consuming -> free; releasing a free page is
    an error; a slice larger than a page is rejected."""
    a = psi.psi_arena_create(desc(1, 0.25, 2))
    try:
        host = np.zeros(4096, np.uint8)
        p0 = psi.psi_page_submit(a, host, 4096)
        p1 = psi.psi_page_submit(a, host, 4096)
        assert (p0, p1) == (0, 1)
        with pytest.raises(psi.PsiError) as e:
            psi.psi_page_submit(a, host, 4096)
        assert e.value.status == psi.PSI_E_PAGE_BUSY
        psi.psi_page_acquire(a, p0)
        psi.psi_page_release(a, p0)
        with pytest.raises(psi.PsiError) as e:
            psi.psi_page_release(a, p0)
        assert e.value.status == psi.PSI_E_STATE
        assert psi.psi_page_submit(a, host, 4096) == 0  # round robin reuses slot 0
        with pytest.raises(psi.PsiError) as e:
            psi.psi_page_submit(a, np.zeros(MiB, np.uint8), MiB)
        assert e.value.status == psi.PSI_E_PAGE_TOO_SMALL
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 3 and s.bytes_h2d == 3 * 4096
    finally:
        psi.psi_arena_destroy(a)


def test_ffn_streams_every_page_once_dry_run():
    """Page reuse across token chunks ([PSI] sec. II-B eq. (2)): with 4
    chunks of 1,024 tokens each U_J and V_J page is copied exactly once (32
    pages = 256 MiB of weights, plus the bias slices), never once per chunk;
    every chunk runs its own up- and down-projection launch (16 tiles x 4
    chunks x 2), and the hidden tile holds one chunk's rows."""
    a = psi.psi_arena_create(desc(80, 8, 2, 8))
    try:
        U, V = cfg5_ffn()
        fake = 0x10000  # device pointers are not touched in a dry run
        psi.psi_ffn_paged(a, fake, 4096, 4096, U, V, 4, fake, fake, psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 32
        assert s.bytes_h2d == 256 * MiB + 16384 * 2 + 4096 * 2
        assert s.kernel_launches == 16 * 4 * 2
        assert s.scratch_high_water == 1024 * 1024 * 2
        psi.psi_arena_reset_stats(a)
        psi.psi_ffn_paged(a, fake, 4096, 4096, U, V, 1, fake, fake, psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 32 and s.kernel_launches == 32
        assert s.scratch_high_water == 4096 * 1024 * 2
    finally:
        psi.psi_arena_destroy(a)


def test_ffn_token_chunks_bound_scratch_dry_run():
    """The hidden tile is sized from one token chunk, so the FFN's scratch
    stays bounded at any token count ([PSI] sec. II-A eq. (1)).  In the
    benchmark's arena (80 MiB: seven 8 MiB pages, no workspace, about 23.9
    MiB of scratch) the FFN of 16,384 tokens is refused in one chunk (32 MiB
    hidden tile) and fits in two or more; ragged chunk counts round the
    chunk up; several chunks need two page slots unless the weights are
    resident."""
    U, V = cfg5_ffn()
    d = desc(80, 8, 7, 0)
    assert psi.psi_ffn_plan(d, 16384, 4096, U, V, token_chunks=1)[0] == psi.PSI_E_SCRATCH_EXHAUSTED
    for chunks, rows in ((2, 8192), (3, 5462), (16, 1024), (16384, 1), (20000, 1)):
        assert psi.psi_ffn_plan(d, 16384, 4096, U, V, token_chunks=chunks) == \
            (psi.PSI_OK, -(-rows * 1024 * 2 // 256) * 256)
    assert psi.psi_ffn_plan(desc(80, 8, 1, 0), 4096, 4096, U, V, token_chunks=2)[0] == psi.PSI_E_INVALID
    Ur = psi.make_matrix(0x1000, 0x2000, 16384, 4096, psi.PSI_SPLIT_ROWS, 1024, 1)
    Vr = psi.make_matrix(0x1000, 0x2000, 4096, 16384, psi.PSI_SPLIT_COLS, 1024, 1)
    assert psi.psi_ffn_plan(desc(80, 8, 1, 0), 4096, 4096, Ur, Vr, token_chunks=2) == \
        (psi.PSI_OK, 2048 * 1024 * 2)


def test_stack_16384_tokens_plans_in_benchmark_arena_dry_run():
    """The 8-block stack at 16,384 tokens (twice the benchmarked count) runs
    inside the same 80 MiB arena of seven pages once the FFN uses two token
    chunks: attention keeps its head-group outputs, K and V^T in the
    caller's accumulator memory (no arena scratch) and the FFN's hidden tile
    is 16 MiB.  In one chunk it is refused before anything is enqueued."""
    Wq, Wk, Wv, _ = cfg5_attn()
    Wo_t = fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, 1024)
    U, V = cfg5_ffn()
    bw = psi.psi_block_weights(Wq, Wk, Wv, Wo_t, U, V)
    a = psi.psi_arena_create(desc(80, 8, 7, 0))
    try:
        with pytest.raises(psi.PsiError) as e:
            psi.psi_block_paged(a, 0x10000, None, 16384, 32, 128, bw, 1, 0x30000, None, 0)
        assert e.value.status == psi.PSI_E_SCRATCH_EXHAUSTED
        assert psi.psi_arena_stats(a).page_copies == 0
        for _ in range(8):
            psi.psi_block_paged(a, 0x10000, None, 16384, 32, 128, bw, 2, 0x30000, None, 0)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 8 * 48
        assert s.scratch_high_water == 8192 * 1024 * 2
        assert s.arena_bytes == 80 * MiB
    finally:
        psi.psi_arena_destroy(a)


def test_output_overlap_rules_dry_run():
    """The projection reads x in every page launch while earlier launches
    have written y, so y must not overlap x.  The FFN, attention and block
    write each element after every read of it: y may be x itself, but not a
    partly overlapping range.  Refusals happen before anything is enqueued."""
    a = psi.psi_arena_create(desc(8, 1, 2, 0))
    try:
        M, K = 64, 256
        W = fake_matrix(256, 256, psi.PSI_SPLIT_ROWS, 128)
        base = 0x100000
        for y in (base, base + 2 * K * 16):
            with pytest.raises(psi.PsiError) as e:
                psi.psi_linear_paged(a, base, M, K, W, None, y, psi.PSI_OP_RESIDUAL)
            assert e.value.status == psi.PSI_E_INVALID
        psi.psi_linear_paged(a, base, M, K, W, None, base + M * K * 2, 0)  # adjacent: fine
        U = fake_matrix(512, 256, psi.PSI_SPLIT_ROWS, 256)
        V = fake_matrix(256, 512, psi.PSI_SPLIT_COLS, 256)
        psi.psi_ffn_paged(a, base, M, K, U, V, 2, None, base, psi.PSI_OP_RESIDUAL)
        with pytest.raises(psi.PsiError) as e:
            psi.psi_ffn_paged(a, base, M, K, U, V, 2, None, base + 16, psi.PSI_OP_RESIDUAL)
        assert e.value.status == psi.PSI_E_INVALID
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 2 + 4
    finally:
        psi.psi_arena_destroy(a)
    Wq, Wk, Wv, Wo = cfg5_attn()
    U, V = cfg5_ffn()
    bw = psi.psi_block_weights(Wq, Wk, Wv, Wo, U, V)
    a = psi.psi_arena_create(desc(80, 8, 2, 8))
    try:
        with pytest.raises(psi.PsiError) as e:
            psi.psi_block_paged(a, 0x10000, 0x10000 + 4096, 8192, 32, 128, bw, 1, 0x30000, None, 0)
        assert e.value.status == psi.PSI_E_INVALID
        assert psi.psi_arena_stats(a).page_copies == 0
    finally:
        psi.psi_arena_destroy(a)


def test_attention_page_order_dry_run():
    """Self- plus cross-attention with 8-head groups: 4 pages per group per
    sub-block, 32 pages = 256 MiB for the two sub-blocks."""
    a = psi.psi_arena_create(desc(80, 8, 2, 8))
    try:
        Wq, Wk, Wv, Wo = cfg5_attn()
        fake = 0x10000
        psi.psi_attn_paged(a, fake, 6144, None, 0, 32, 128, Wq, Wk, Wv, Wo, fake, fake,
                           psi.PSI_OP_RESIDUAL)
        psi.psi_attn_paged(a, fake, 6144, fake, 1024, 32, 128, Wq, Wk, Wv, Wo, fake, fake,
                           psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 32
        assert s.bytes_h2d == 256 * MiB + 2 * (4 * 4096 * 2)
        assert s.kernel_launches == 2 * 4 * 5  # 4 GEMMs + 1 attention per group
        assert s.scratch_high_water == 3 * 6144 * 1024 * 2
    finally:
        psi.psi_arena_destroy(a)


def test_attention_kernel_choice_checked_first_dry_run():
    """PSI_OP_ATTN_CONFIG(c): 0-4 accepted, anything else refused before any
    page copy or launch, for the attention operators and the block driver."""
    a = psi.psi_arena_create(desc(80, 8, 2, 8))
    try:
        Wq, Wk, Wv, Wo = cfg5_attn()
        fake = 0x10000
        for c in range(5):
            psi.psi_attn_paged(a, fake, 6144, None, 0, 32, 128, Wq, Wk, Wv, Wo, fake, fake,
                               psi.PSI_OP_RESIDUAL | psi.PSI_OP_ATTN_CONFIG(c))
        s0 = psi.psi_arena_stats(a)
        for c in (5, 7):
            with pytest.raises(psi.PsiError) as e:
                psi.psi_attn_paged(a, fake, 6144, None, 0, 32, 128, Wq, Wk, Wv, Wo, fake, fake,
                                   psi.PSI_OP_RESIDUAL | psi.PSI_OP_ATTN_CONFIG(c))
            assert e.value.status == psi.PSI_E_INVALID
        U, V = cfg5_ffn()
        bw = psi.psi_block_weights(Wq, Wk, Wv, Wo, U, V)
        with pytest.raises(psi.PsiError) as e:
            psi.psi_block_paged(a, 0x10000, None, 8192, 32, 128, bw, 1, 1 << 40, None, psi.PSI_OP_ATTN_CONFIG(6))
        assert e.value.status == psi.PSI_E_INVALID
        s1 = psi.psi_arena_stats(a)
        assert (s1.page_copies, s1.kernel_launches) == (s0.page_copies, s0.kernel_launches)
    finally:
        psi.psi_arena_destroy(a)


def test_checkpoint_size_independence_dry_run():
    """[PSI] sec. II-A: the managed footprint does not depend on checkpoint
    size -- stacks of 2, 4 and 8 blocks give the same arena peak and scratch
    high-water mark; only the bytes streamed grow."""
    peaks, streamed = [], []
    for nblocks in (2, 4, 8):
        a = psi.psi_arena_create(desc(80, 8, 2, 8))
        try:
            Wq, Wk, Wv, Wo = cfg5_attn()
            U, V = cfg5_ffn()
            bw = psi.psi_block_weights(Wq, Wk, Wv, Wo, U, V)
            for _ in range(nblocks):
                psi.psi_block_paged(a, 0x10000, 1 << 40, 8192, 32, 128, bw, 1, 0x30000, None, 0)
            s = psi.psi_arena_stats(a)
            peaks.append((s.arena_bytes, s.scratch_high_water))
            streamed.append(s.bytes_h2d)
        finally:
            psi.psi_arena_destroy(a)
    assert peaks[0] == peaks[1] == peaks[2]
    assert streamed[1] == 2 * streamed[0] and streamed[2] == 4 * streamed[0]


def test_single_hip_runtime_in_process():
    """The library binds to the HIP runtime of the process (torch's copy),
    so torch's streams and the library's are one runtime's streams."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().splitlines()
    hip = {l.split()[-1] for l in maps if "libamdhip64" in l}
    hsa = {l.split()[-1] for l in maps if "libhsa-runtime64" in l}
    assert len(hip) == 1, hip
    assert len(hsa) <= 1, hsa


def test_trace_needs_profiling_arena():
    """psi_arena_trace_start / _read reject an arena created without
    PSI_ARENA_PROFILE, and accept a profiling one (dry run: no events)."""
    a = psi.psi_arena_create(desc(8, 1, 2))
    try:
        with pytest.raises(psi.PsiError):
            psi.psi_arena_trace_start(a, 16)
        with pytest.raises(psi.PsiError):
            psi.psi_arena_trace_read(a, 16)
        with pytest.raises(psi.PsiError):
            psi.psi_arena_set_timing(a, False)
    finally:
        psi.psi_arena_destroy(a)
    a = psi.psi_arena_create(desc(8, 1, 2, flags=psi.PSI_ARENA_DRY_RUN | psi.PSI_ARENA_PROFILE))
    try:
        psi.psi_arena_trace_start(a, 16)
        assert psi.psi_arena_trace_read(a, 16) == []
        psi.psi_arena_set_timing(a, False)
        psi.psi_arena_set_timing(a, True)
    finally:
        psi.psi_arena_destroy(a)


def test_ffn_tiled_plans_and_recompute_stream_dry_run():
    """FFN over down-projection output tiles ([PSI] sec. III-B): plan checks,
    and the recompute baseline streams every U_J page again for every output
    tile while the output-tile page of V stays held (two page slots)."""
    d = desc(80, 8, 2, 8)
    U, _ = cfg5_ffn()                                            # [16384, 4096], 1,024-row pages
    Vo = fake_matrix(4096, 16384, psi.PSI_SPLIT_ROWS, 256)       # 256 x 16,384 = 8 MiB pages
    st, need = psi.psi_ffn_tiled_plan(d, 2048, 4096, U, Vo, psi.PSI_FFN_REUSE)
    assert st == psi.PSI_OK and need == 2 * 2048 * 1024 * 2 + 2048 * 256 * 4  # two hidden-tile buffers
    st, need = psi.psi_ffn_tiled_plan(d, 2048, 4096, U, Vo, psi.PSI_FFN_RECOMPUTE)
    assert st == psi.PSI_OK and need == 2048 * 1024 * 2 + 2048 * 256 * 4
    assert psi.psi_ffn_tiled_plan(d, 2048, 4096, U, Vo, 3)[0] == psi.PSI_E_INVALID
    Vk = fake_matrix(4096, 16384, psi.PSI_SPLIT_COLS, 1024)
    assert psi.psi_ffn_tiled_plan(d, 2048, 4096, U, Vk, psi.PSI_FFN_REUSE)[0] == psi.PSI_E_INVALID
    Vbig = fake_matrix(4096, 16384, psi.PSI_SPLIT_ROWS, 512)     # 16 MiB pages
    assert psi.psi_ffn_tiled_plan(d, 2048, 4096, U, Vbig, psi.PSI_FFN_REUSE)[0] == psi.PSI_E_PAGE_TOO_SMALL
    one = desc(80, 8, 1, 8)
    assert psi.psi_ffn_tiled_plan(one, 2048, 4096, U, Vo, psi.PSI_FFN_RECOMPUTE)[0] == psi.PSI_E_INVALID
    assert psi.psi_ffn_tiled_plan(one, 2048, 4096, U, Vo, psi.PSI_FFN_REUSE)[0] == psi.PSI_OK
    a = psi.psi_arena_create(desc(80, 8, 3, 0))
    try:
        fake = 0x10000
        with pytest.raises(psi.PsiError) as e:  # FFN reuse without a journal
            psi.psi_ffn_tiled(a, fake, 512, 4096, U, Vo, psi.PSI_FFN_REUSE, None, 0, 0, fake)
        assert e.value.status == psi.PSI_E_INVALID
        with pytest.raises(psi.PsiError) as e:  # y aliasing x over 16 output tiles
            psi.psi_ffn_tiled(a, fake, 512, 4096, U, Vo, psi.PSI_FFN_RECOMPUTE, None, 0, 0, fake)
        assert e.value.status == psi.PSI_E_INVALID
        psi.psi_ffn_tiled(a, fake, 512, 4096, U, Vo, psi.PSI_FFN_RECOMPUTE, None, 0, 0, 1 << 40)
        s = psi.psi_arena_stats(a)
        n_o, n_j = 4096 // 256, 16384 // 1024
        assert s.page_copies == n_o * (1 + n_j)
        assert s.kernel_launches == n_o * n_j * 2  # up + down per (output tile, hidden tile)
    finally:
        psi.psi_arena_destroy(a)


def test_attn_ext_plan_errors():
    """Query/key normalisation-rotary settings are checked by the plan."""
    ms = [fake_matrix(256, 256, psi.PSI_SPLIT_ROWS, 128) for _ in range(3)] + \
         [fake_matrix(256, 256, psi.PSI_SPLIT_COLS, 128)]
    d = desc(8, 1)
    ok = psi.qk_norm_rope(0x1000, None, 1e-6)
    st, need = psi.psi_attn_ext_plan(d, 64, 0, 4, 64, *ms, ok)
    assert st == psi.PSI_OK and need >= (64 + 64) * 256 * 2
    assert psi.psi_attn_plan(d, 64, 0, 4, 64, *ms)[0] == psi.PSI_OK  # 64-dim heads
    assert psi.psi_attn_plan(d, 64, 0, 8, 32, *ms)[0] == psi.PSI_E_INVALID
    bad = [psi.qk_norm_rope(0x1000, None, 0.0),                  # eps <= 0 with a gamma
           psi.qk_norm_rope(0x1000, None, 1e-6, norm_tile=12),   # not a multiple of 8
           psi.qk_norm_rope(None, None, 1e-6, cos_q=0x1000),     # sin_q missing
           psi.qk_norm_rope(None, None, 1e-6, cos_k=0x1000, sin_k=0x1000)]  # key tables alone
    for s in bad:
        assert psi.psi_attn_ext_plan(d, 64, 0, 4, 64, *ms, s)[0] == psi.PSI_E_INVALID
    s = psi.qk_norm_rope(None, None, 1e-6, cos_q=0x1000, sin_q=0x1000)
    assert psi.psi_attn_ext_plan(d, 64, 32, 4, 64, *ms, s)[0] == psi.PSI_E_INVALID  # Mk != M
    s = psi.qk_norm_rope(None, None, 1e-6, cos_q=0x1008, sin_q=0x1000)
    assert psi.psi_attn_ext_plan(d, 64, 0, 4, 64, *ms, s)[0] == psi.PSI_E_ALIGN


def test_attn_ext_audio_shape_dry_run():
    """Audio self-attention (126 tokens, 32 heads of 64) with 8-head pages:
    16 pages, 4 GEMMs and one attention per group plus one
    normalisation-rotary launch each for Q and K; biases and both gammas
    share the operator's bias request."""
    d, M, gw = 2048, 126, 512
    ms = [fake_matrix(d, d, psi.PSI_SPLIT_ROWS, gw) for _ in range(3)] + \
         [fake_matrix(d, d, psi.PSI_SPLIT_COLS, gw)]
    a = psi.psi_arena_create(desc(16, 2))
    try:
        nr = psi.qk_norm_rope(0x1000, 0x2000, 1e-6, 0, 0x3000, 0x4000)
        fake = 0x10000
        psi.psi_attn_paged_ext(a, fake, M, None, 0, 32, 64, *ms, nr, fake, fake, psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 16
        assert s.bytes_h2d == 16 * gw * d * 2 + 6 * d * 2
        assert s.kernel_launches == 4 * 5 + 2
        ldvt = 128
        assert s.scratch_high_water == 2 * M * d * 2 + gw * ldvt * 2
    finally:
        psi.psi_arena_destroy(a)


def test_attn_tiled_plan_and_lowlive_block_dry_run():
    """Low-live-state block ([PSI] sec. III-B: state retained on device or in
    the host journal): Wo and V split by rows into output tiles; the arena
    holds two [M, gw] buffers plus max(K/V^T, ACC_o) for attention and two
    hidden tiles plus ACC_o for the FFN; pages stream once per block."""
    d, h, M, gw, to_a, to_f, th = 4096, 16384, 2048, 1024, 512, 256, 1024
    q, k, v = [fake_matrix(d, d, psi.PSI_SPLIT_ROWS, gw) for _ in range(3)]
    wo = fake_matrix(d, d, psi.PSI_SPLIT_ROWS, to_a)
    st, need = psi.psi_attn_tiled_plan(desc(80, 8, 2), M, 0, 32, 128, q, k, v, wo)
    ldvt = M
    kv = M * gw * 2 + gw * ldvt * 2
    assert st == psi.PSI_OK and need == 2 * M * gw * 2 + max(kv, M * to_a * 4)
    wo_cols = fake_matrix(d, d, psi.PSI_SPLIT_COLS, gw)
    assert psi.psi_attn_tiled_plan(desc(80, 8, 2), M, 0, 32, 128, q, k, v, wo_cols)[0] == psi.PSI_E_INVALID
    U = fake_matrix(h, d, psi.PSI_SPLIT_ROWS, th)
    V = fake_matrix(d, h, psi.PSI_SPLIT_ROWS, to_f)
    bw = psi.psi_block_weights(q, k, v, wo, U, V)
    a = psi.psi_arena_create(desc(80, 8, 2))
    try:
        fake, fake_journal = 0x10000, 0x20000
        psi.psi_block_lowlive(a, fake, M, 32, 128, bw, fake_journal, 0)
        s = psi.psi_arena_stats(a)
        nG, nOa, nJ, nOf = d // gw, d // to_a, h // th, d // to_f
        assert s.page_copies == 3 * nG + nOa + nJ + nOf
        assert s.kernel_launches == 4 * nG + nOa * nG + nJ + nOf * nJ
        assert s.bytes_h2d == 4 * d * d * 2 + 2 * d * h * 2 + (4 * d + h + d) * 2
        assert s.scratch_high_water == max(need, 2 * M * th * 2 + M * to_f * 4)
    finally:
        psi.psi_arena_destroy(a)


def test_new_entry_points_empty_inputs_and_layout_errors_dry_run():
    """Zero tokens enqueue nothing; a low-live block needs Wo and V split by
    rows (output tiles), and the extended attention rejects a gain block that
    does not fit the bias slot together with the biases."""
    d, h, gw = 512, 2048, 128
    q, k, v = [fake_matrix(d, d, psi.PSI_SPLIT_ROWS, gw) for _ in range(3)]
    wo_rows = fake_matrix(d, d, psi.PSI_SPLIT_ROWS, 128)
    wo_cols = fake_matrix(d, d, psi.PSI_SPLIT_COLS, gw)
    U = fake_matrix(h, d, psi.PSI_SPLIT_ROWS, 256)
    V_rows = fake_matrix(d, h, psi.PSI_SPLIT_ROWS, 128)
    a = psi.psi_arena_create(desc(16, 1))
    try:
        fake, fj = 0x10000, 0x20000
        nr = psi.qk_norm_rope(0x1000, 0x2000, 1e-6)
        psi.psi_attn_paged_ext(a, fake, 0, None, 0, 4, 128, q, k, v, wo_cols, nr, None, fake, 0)
        psi.psi_attn_tiled(a, fake, 0, None, 0, 4, 128, q, k, v, wo_rows, fj, 0, 0, fake, 0)
        psi.psi_block_lowlive(a, fake, 0, 4, 128, psi.psi_block_weights(q, k, v, wo_rows, U, V_rows), fj, 0)
        s = psi.psi_arena_stats(a)
        assert s.kernel_launches == 0 and s.page_copies == 0
        for bad in (psi.psi_block_weights(q, k, v, wo_cols, U, V_rows),
                    psi.psi_block_weights(q, k, v, wo_rows, U, fake_matrix(d, h, psi.PSI_SPLIT_COLS, 256))):
            with pytest.raises(psi.PsiError) as e:
                psi.psi_block_lowlive(a, fake, 64, 4, 128, bad, fj, 0)
            assert e.value.status == psi.PSI_E_INVALID
        with pytest.raises(psi.PsiError) as e:  # the head-group outputs need a journal
            psi.psi_attn_tiled(a, fake, 64, None, 0, 4, 128, q, k, v, wo_rows, None, 0, 0, fake, 0)
        assert e.value.status == psi.PSI_E_INVALID
    finally:
        psi.psi_arena_destroy(a)
    # biases (4 x 1 KiB) and two 1 KiB gains in a 4 KiB bias slot
    small = psi.arena_desc(16 * MiB, 1 * MiB, 2, 0, 4096, None, psi.PSI_ARENA_DRY_RUN)
    st, _ = psi.psi_attn_ext_plan(small, 64, 0, 4, 128, q, k, v, wo_cols, psi.qk_norm_rope(0x1000, 0x2000, 1e-6))
    assert st == psi.PSI_E_PAGE_TOO_SMALL
    assert psi.psi_attn_ext_plan(small, 64, 0, 4, 128, q, k, v, wo_cols, None)[0] == psi.PSI_OK


def test_attention_output_tiles_plan_and_page_order_dry_run():
    """With Wo split by rows (output tiles) the O-projection runs once per
    tile over the full K after every head group, from the groups' outputs
    kept in acc_dev's memory, which also takes K and V^T of one group where
    they fit behind them: the stack's attention needs no arena scratch, the
    same 16 pages stream, Wo's last, and PSI_OP_STORE_ACC (no fp32
    accumulator exists) and a misaligned acc_dev are refused.  Without
    acc_dev the outputs take M x d BF16 of scratch."""
    Wq, Wk, Wv, _ = cfg5_attn()
    Wo_t = fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, 768)  # ragged: 5 tiles of 768 + 256
    d5 = desc(80, 8, 5, 0)
    # O (64 MiB), K and V^T (32 MiB) all sit in acc_dev's 128 MiB
    st, need = psi.psi_attn_plan(desc(80, 8, 8, 0), 8192, 0, 32, 128, Wq, Wk, Wv, Wo_t, True)
    assert st == psi.PSI_OK and need == 0
    # cross-attention to 16,384 keys: K and V^T (64 MiB) do not fit behind O of 4,096 queries
    st, need = psi.psi_attn_plan(desc(160, 8, 5, 0), 4096, 16384, 32, 128, Wq, Wk, Wv, Wo_t, True)
    assert st == psi.PSI_OK and need == 2 * 16384 * 1024 * 2
    st, _ = psi.psi_attn_plan(d5, 8192, 0, 32, 128, *cfg5_attn(), True)
    assert st == psi.PSI_E_SCRATCH_EXHAUSTED  # the K-split keeps Q_g, K_g, V_g^T in the arena
    st, need = psi.psi_attn_plan(desc(80, 8, 2, 0), 1024, 0, 32, 128, Wq, Wk, Wv, Wo_t, False)
    assert st == psi.PSI_OK and need == 2 * 1024 * 1024 * 2 + 1024 * 4096 * 2
    a = psi.psi_arena_create(d5)
    try:
        fake = 0x10000
        psi.psi_attn_paged(a, fake, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_t, fake, fake,
                           psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 12 + 6
        assert s.bytes_h2d == 16 * 8 * MiB + 4 * 4096 * 2
        assert s.kernel_launches == 4 * 4 + 6  # Q, K, V^T, attention per group; one GEMM per tile
        assert s.scratch_high_water == 0       # O, K and V^T in acc_dev's memory
        with pytest.raises(psi.PsiError) as e:
            psi.psi_attn_paged(a, fake, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_t, fake + 8, fake, 0)
        assert e.value.status == psi.PSI_E_ALIGN
        with pytest.raises(psi.PsiError) as e:
            psi.psi_attn_paged(a, fake, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_t, fake, fake,
                               psi.PSI_OP_STORE_ACC)
        assert e.value.status == psi.PSI_E_INVALID
        Wo_bad = fake_matrix(4096, 4096, psi.PSI_SPLIT_COLS, 512)  # a K-split Wo needs the group block
        with pytest.raises(psi.PsiError) as e:
            psi.psi_attn_paged(a, fake, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_bad, fake, fake, 0)
        assert e.value.status == psi.PSI_E_INVALID
    finally:
        psi.psi_arena_destroy(a)


def test_block_copies_ffn_pages_during_attention_dry_run():
    """psi_block_paged hands the FFN's page requests to the attention
    sub-block's feeder: once every attention page is submitted, page slots
    freed by attention kernels take the FFN's first pages, and the FFN's
    feeder adopts them.  Every page is still copied exactly once per block
    (48 in the benchmarked layout), blocks in a row stay consistent, and
    the two operators called on their own copy nothing ahead."""
    Wq, Wk, Wv, _ = cfg5_attn()
    Wo_t = fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, 1024)
    U, V = cfg5_ffn()
    bw = psi.psi_block_weights(Wq, Wk, Wv, Wo_t, U, V)
    a = psi.psi_arena_create(desc(80, 8, 7, 0))
    try:
        for n in range(1, 4):
            psi.psi_block_paged(a, 0x10000, None, 8192, 32, 128, bw, 1, 0x30000, None, 0)
            s = psi.psi_arena_stats(a)
            assert s.page_copies == 48 * n
            assert 0 < s.ahead_page_copies <= 32 * n
            assert s.ahead_page_copies % n == 0 and s.ahead_page_copies // n <= 7 + 9
        psi.psi_arena_reset_stats(a)
        psi.psi_attn_paged(a, 0x10000, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_t, 0x30000, 0x10000,
                           psi.PSI_OP_RESIDUAL)
        psi.psi_ffn_paged(a, 0x10000, 8192, 4096, U, V, 1, 0x30000, 0x10000, psi.PSI_OP_RESIDUAL)
        s = psi.psi_arena_stats(a)
        assert s.page_copies == 48 and s.ahead_page_copies == 0
    finally:
        psi.psi_arena_destroy(a)


def test_scratch_lent_as_page_slots_dry_run():
    """An operator lends the whole pages of scratch above its own allocations
    as page slots for its requests: in the stack's 80 MiB arena (7 pages),
    attention with output tiles (no arena scratch) lends two 8 MiB slots,
    while the FFN, whose 16 MiB hidden tile leaves less than a page, lends
    none; a sync-copy arena lends none.  Copies, launches and the scratch
    high-water mark are unchanged."""
    Wq, Wk, Wv, _ = cfg5_attn()
    Wo_t = fake_matrix(4096, 4096, psi.PSI_SPLIT_ROWS, 1024)
    U, V = cfg5_ffn()
    fake = 0x10000
    for flags, lent_attn in ((psi.PSI_ARENA_DRY_RUN, True),
                             (psi.PSI_ARENA_DRY_RUN | psi.PSI_ARENA_SYNC_COPY, False)):
        a = psi.psi_arena_create(desc(80, 8, 7, 0, flags))
        try:
            psi.psi_attn_paged(a, fake, 8192, None, 0, 32, 128, Wq, Wk, Wv, Wo_t, fake, fake,
                               psi.PSI_OP_RESIDUAL)
            s = psi.psi_arena_stats(a)
            assert s.page_copies == 16 and s.kernel_launches == 20 and s.scratch_high_water == 0
            assert (s.lent_page_copies > 0) == lent_attn
            lent0 = s.lent_page_copies
            psi.psi_ffn_paged(a, fake, 8192, 4096, U, V, 1, fake, fake, psi.PSI_OP_RESIDUAL)
            s = psi.psi_arena_stats(a)
            assert s.page_copies == 48 and s.lent_page_copies == lent0
            assert s.scratch_high_water == 8192 * 1024 * 2
        finally:
            psi.psi_arena_destroy(a)


def test_pack_tiles_layout():
    """PSI_SPLIT_TILES page image: row tiles in order, each row tile's column
    blocks in order, each page a contiguous row-major block (ragged last row
    tile and column block); page counts and sizes follow."""
    rows, cols, br, bc = 10, 24, 4, 16
    W = np.arange(rows * cols, dtype=np.uint16).reshape(rows, cols)
    img = np.empty(rows * cols, np.uint16)
    psi.psi_pack_tiles(W, rows, cols, br, bc, img)
    expect = np.concatenate([W[r0:r0 + br, c0:c0 + bc].ravel() for r0 in range(0, rows, br)
                             for c0 in range(0, cols, bc)])
    assert np.array_equal(img, expect)
    m = psi.make_matrix(img, None, rows, cols, psi.PSI_SPLIT_TILES, br, 0, bc)
    assert psi.psi_matrix_pages(m) == 3 * 2
    sizes = [psi.psi_matrix_page_bytes(m, p) for p in range(6)]
    assert sizes == [4 * 16 * 2, 4 * 8 * 2, 4 * 16 * 2, 4 * 8 * 2, 2 * 16 * 2, 2 * 8 * 2]
    assert sum(sizes) == rows * cols * 2
    with pytest.raises(psi.PsiError):
        psi.psi_pack_tiles(W, rows, cols, br, bc, W)  # in place is refused


def test_lowlive_hidden_state_is_the_journal_figure():
    """[PSI] sec. IV-C prints a per-block journal figure (tests/golden).  It
    factors as one BF16 FFN hidden state of 4,991 tokens at width 16,384, the
    token count of the low-live workload, whose tiled FFN commits exactly that
    many bytes of hidden tiles per block (16 tiles of 4,991 x 1,024)."""
    fig = golden.values("journal_block_bytes.txt")["bytes_per_block"]
    M, h, th = 4991, 16384, 1024
    assert fig == M * h * 2
    assert fig == (h // th) * M * th * 2


def test_two_d_page_tiles_rules_and_lowlive_traffic_dry_run():
    """2-D page tiles serve only the output-tile schedules: the projection,
    the paged attention and the paged FFN refuse them; the tiled FFN needs
    whole hidden tiles per page and the tiled attention whole head groups.
    In a low-live block, output tiles of 1,024 (FFN, 4 pages each) and 2,048
    rows (attention, 2 pages each) stream the same pages as narrow tiles but
    reload each hidden state 4 times instead of 16 and each head-group output
    2 times instead of 8 ([PSI] sec. IV-C quantifies this journal traffic)."""
    d, h, M, gw, th = 4096, 16384, 4991, 1024, 1024
    T = lambda r, c, br, bc: psi.make_matrix(0x1000, 0x2000, r, c, psi.PSI_SPLIT_TILES, br, 0, bc)
    dsc = desc(80, 8, 2)
    q, k, v = [fake_matrix(d, d, psi.PSI_SPLIT_ROWS, gw) for _ in range(3)]
    U = fake_matrix(h, d, psi.PSI_SPLIT_ROWS, th)
    Vt, Wot = T(d, h, 1024, 4096), T(d, d, 2048, 2048)
    assert psi.psi_linear_plan(dsc, 64, d, Wot)[0] == psi.PSI_E_INVALID
    assert psi.psi_attn_plan(dsc, 64, 0, 32, 128, q, k, v, Wot)[0] == psi.PSI_E_INVALID
    assert psi.psi_ffn_tiled_plan(dsc, M, d, U, T(d, h, 1024, 3072), psi.PSI_FFN_REUSE)[0] == psi.PSI_OK
    assert psi.psi_ffn_tiled_plan(dsc, M, d, U, T(d, h, 1024, 2040), psi.PSI_FFN_REUSE)[0] == psi.PSI_E_INVALID
    assert psi.psi_ffn_tiled_plan(dsc, M, d, U, T(d, h, 1024, 8192), psi.PSI_FFN_REUSE)[0] == \
        psi.PSI_E_PAGE_TOO_SMALL
    assert psi.psi_attn_tiled_plan(dsc, M, 0, 32, 128, q, k, v, T(d, d, 2048, 1536))[0] == psi.PSI_E_INVALID
    st, need_f = psi.psi_ffn_tiled_plan(dsc, M, d, U, Vt, psi.PSI_FFN_REUSE)
    assert st == psi.PSI_OK and need_f == 2 * (-(-M * th * 2 // 256) * 256) + -(-M * 1024 * 4 // 256) * 256
    st, need_a = psi.psi_attn_tiled_plan(dsc, M, 0, 32, 128, q, k, v, Wot)
    assert st == psi.PSI_OK
    counts = {}
    for name, Wo, V in (("rows", fake_matrix(d, d, psi.PSI_SPLIT_ROWS, 512), fake_matrix(d, h, psi.PSI_SPLIT_ROWS, 256)),
                        ("tiles", Wot, Vt)):
        a = psi.psi_arena_create(dsc)
        try:
            psi.psi_block_lowlive(a, 0x10000, M, 32, 128, psi.psi_block_weights(q, k, v, Wo, U, V), 0x20000, 0)
            s = psi.psi_arena_stats(a)
            counts[name] = (s.page_copies, s.bytes_h2d, s.kernel_launches)
        finally:
            psi.psi_arena_destroy(a)
    nG, nJ = d // gw, h // th
    weights = 4 * d * d * 2 + 2 * d * h * 2 + (4 * d + h + d) * 2
    assert counts["rows"][:2] == (3 * nG + 8 + nJ + 16, weights)  # Wo in 8 pages of 4 MiB
    assert counts["tiles"][:2] == (3 * nG + 4 + nJ + 16, weights)  # Wo in 4 pages of 8 MiB
    # GEMMs: per group Q, K, V^T (+ attention); O-projection one per (row tile, group);
    # FFN one up per hidden tile and one down per (row tile, hidden tile)
    assert counts["rows"][2] == 4 * nG + 8 * nG + nJ + 16 * nJ
    assert counts["tiles"][2] == 4 * nG + 2 * nG + nJ + 4 * nJ
