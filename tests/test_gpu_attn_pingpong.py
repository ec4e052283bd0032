"""The attention kernels against each other, bit for bit, through the C ABI.

PSI_OP_ATTN_CONFIG(c) selects the kernel: 1 = 128-query workgroups, 2 =
256-query workgroups, 3 = 256-query software-pipelined with the waves in lock
step, 4 = 256-query ping-pong (the two wave groups of a workgroup alternate
softmax and matrix phases); 0 is the automatic choice, which takes the
ping-pong kernel over 512 or more keys or 256 or more workgroups of 256
queries.  All compute every query's scores, online-softmax updates and P.V
accumulation in the same order, so their outputs are compared bit for bit:
self- and cross-attention with ragged query and key counts, large and small
grids, head dimensions 128 and 64, and the three softmax-weight precisions
(fp32 weights as three BF16 terms, two terms, BF16 numerator weights).
Parity with the oracle at the benchmark's shape, where the ping-pong kernel
runs, is checked by the full-size tests.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023); attention
sub-block of sec. II-B, softmax weights of sec. III-A.
"""
import numpy as np
import pytest

from memory_bounded_weight_amd import synth
from tests.gpu_util import dev, empty_bf16, f, host, make_arena

pytestmark = pytest.mark.gpu

KiB = 1024


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def matrices(P, w, gw):
    return (P.pinned_matrix(w["Wq"], w["bq"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wk"], w["bk"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wv"], w["bv"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_COLS, gw))


def run(P, x, ctx, ms, heads, dh, flags):
    """psi_attn_paged with every head in one group (one attention launch)."""
    M, d = x.shape
    Mc = 0 if ctx is None else ctx.shape[0]
    Ms = Mc or M
    gw = heads * dh
    pb = gw * d * 2
    ldvt = (Ms + 63) // 64 * 64
    scratch = (M + Ms) * d * 2 + gw * ldvt * 2 + M * d * 4 + 16 * KiB
    ar = make_arena(2 * pb + 2 * 64 * KiB + scratch, pb, 2)
    try:
        xd = dev(x)
        cd = dev(ctx) if ctx is not None else None
        y = empty_bf16(M, d)
        P.psi_attn_paged(ar, xd, M, cd, Mc, heads, dh, *ms, None, y, flags | P.PSI_OP_RESIDUAL)
        P.psi_arena_sync(ar)
        return host(y)
    finally:
        P.psi_arena_destroy(ar)


@pytest.mark.parametrize("dh,heads,M,Mc", [(128, 8, 7990, 0), (128, 8, 7990, 3000),
                                           (64, 16, 7990, 0), (64, 16, 4000, 2999),
                                           (128, 2, 777, 0), (64, 4, 300, 1000), (128, 2, 1000, 513),
                                           (64, 8, 126, 0), (128, 3, 300, 64)])
def test_attention_kernels_bitwise(P, dh, heads, M, Mc):
    rng = np.random.default_rng(1000 + dh + M + Mc)
    d = heads * dh
    x = synth.normal_bf16(rng, (M, d), 1.0)
    ctx = synth.normal_bf16(rng, (Mc, d), 1.0) if Mc else None
    ms = matrices(P, synth.attn_weights(rng, d), d)
    for fl in (0, P.PSI_OP_ATTN_P2, P.PSI_OP_BF16_SOFTMAX):
        y_auto = run(P, x, ctx, ms, heads, dh, fl)
        assert np.isfinite(f(y_auto)).all()
        for c in (1, 2, 3, 4):
            y = run(P, x, ctx, ms, heads, dh, fl | P.PSI_OP_ATTN_CONFIG(c))
            diff = np.flatnonzero(y != y_auto)
            assert diff.size == 0, (f"dh {dh} M {M} Mc {Mc} flags {fl:#x} kernel {c}: {diff.size} outputs "
                                    f"differ, first at {np.unravel_index(diff[0], y.shape)}")


def test_attention_kernel_choice_out_of_range_refused(P):
    rng = np.random.default_rng(5)
    heads, dh = 2, 64
    d = heads * dh
    x = synth.normal_bf16(rng, (64, d), 1.0)
    ms = matrices(P, synth.attn_weights(rng, d), d)
    with pytest.raises(P.PsiError) as e:
        run(P, x, None, ms, heads, dh, P.PSI_OP_ATTN_CONFIG(5))
    assert "PSI_E_INVALID" in str(e.value)
