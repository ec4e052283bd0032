"""Same-input numeric probes of the baseline and modified operator choices
([PSI] sec. III-A "numerical choices", sec. IV-B diagnostics) at the audio
shapes, against the oracle.

* Projection bias: the audio FFN up-projection (126 tokens, 2,048 -> 8,192,
  i.e. 1,032,192 outputs).  Baseline PSI rounds the matrix product to BF16
  and then adds the bias (a second BF16 write); modified PSI adds the bias
  in fp32 before the single write.  Differing BF16 elements are counted
  against the dense single-rounding result.
* Attention numerator: 64-dim-head audio self-attention (126 tokens, 32
  heads, 258,048 outputs).  Baseline: BF16 exponential weights in the
  numerator; modified: fp32 online accumulation (fp32 weights, as three
  BF16 terms on the matrix cores); also the two-term option (about 17-bit
  weights).  The inputs lie on a
  lattice on which the projections are exact in fp32, so the GPU and the
  oracle attend over identical Q, K, V (the paper's identical-input probe);
  O is read from the stage-probe journal.

The counts are printed (run with -s to see them); the assertions check the
direction and size of the effect, which the paper reports as 267,593
differing elements removed and 68,979 -> 45 differing elements.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import numpy as np
import pytest
import torch

import oracle
from memory_bounded_weight_amd import synth
from tests.gpu_util import MiB, assert_bf16_close, dev, empty_bf16, f, host, make_arena

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


def rel_l2(got, ref):
    g, r = f(got).astype(np.float64), f(ref).astype(np.float64)
    return float(np.linalg.norm(g - r) / np.linalg.norm(r))


def report(name, n, **variants):
    parts = [f"{k}: {int(np.count_nonzero(v[0] != v[1]))} differ, rel L2 {rel_l2(*v):.3e}"
             for k, v in variants.items()]
    print(f"\n[probe] {name} ({n} outputs): " + "; ".join(parts))


def test_probe_projection_bias_rounding(P):
    M, K, N = 126, 2048, 8192
    c = synth.linear_case(seed=31, M=M, K=K, N=N)
    W = P.pinned_matrix(c["W"], c["b"], P.PSI_SPLIT_ROWS, 2048)
    ar = make_arena(20 * MiB, 8 * MiB, 2)
    try:
        x = dev(c["x"])
        ys = {}
        for name, fl in (("modified", 0), ("baseline", P.PSI_OP_BASELINE_BIAS)):
            y = empty_bf16(M, N)
            P.psi_linear_paged(ar, x, M, K, W, None, y, fl)
            P.psi_arena_sync(ar)
            ys[name] = host(y)
    finally:
        P.psi_arena_destroy(ar)
    ref = oracle.linear(c["x"], c["W"], c["b"])
    ref_base = oracle.linear(c["x"], c["W"], c["b"], variant=1)
    report("projection bias", M * N, modified=(ys["modified"], ref), baseline=(ys["baseline"], ref))
    # each GPU variant matches the oracle's own variant
    assert_bf16_close(ys["modified"], ref)
    assert_bf16_close(ys["baseline"], ref_base)
    n_mod = int(np.count_nonzero(ys["modified"] != ref))
    n_base = int(np.count_nonzero(ys["baseline"] != ref))
    assert n_mod < M * N // 100, n_mod          # accumulation order only
    assert n_base > 10 * max(n_mod, 1000), (n_base, n_mod)


def test_probe_attention_numerator_64dim(P):
    M, d, heads, dh, gw = 126, 2048, 32, 64, 512
    c = synth.lattice_attn_case(seed=32, M=M, d=d)
    x, w = c["x"], c["w"]
    mats = (P.pinned_matrix(w["Wq"], w["bq"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wk"], w["bk"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wv"], w["bv"], P.PSI_SPLIT_ROWS, gw),
            P.pinned_matrix(w["Wo"], w["bo"], P.PSI_SPLIT_COLS, gw))
    ar = make_arena(16 * MiB, gw * d * 2, 2)
    j = P.psi_journal_create(MiB, 2, 3 * M * d * 2 + MiB)
    Os = {}
    try:
        xd = dev(x)
        for step, (name, fl) in enumerate((("modified", 0), ("two_term", P.PSI_OP_ATTN_P2),
                                           ("baseline", P.PSI_OP_BF16_SOFTMAX))):
            P.psi_arena_set_probe(ar, j, step, 0)
            y = empty_bf16(M, d)
            P.psi_attn_paged(ar, xd, M, None, 0, heads, dh, *mats, None, y, fl | P.PSI_OP_RESIDUAL)
            P.psi_arena_sync(ar)
            P.psi_journal_sync(j)
            parts = []
            for g in range(d // gw):
                o = np.empty((M, gw), np.uint16)
                P.psi_journal_read(j, P.key(step, 0, g, P.PSI_ROLE_ATTN_O), o, o.nbytes)
                parts.append(o)
            Os[name] = np.concatenate(parts, axis=1)
    finally:
        P.psi_arena_set_probe(ar, None)
        P.psi_journal_destroy(j)
        P.psi_arena_destroy(ar)
    Q = oracle.linear(x, w["Wq"], w["bq"])
    K = oracle.linear(x, w["Wk"], w["bk"])
    V = oracle.linear(x, w["Wv"], w["bv"])
    ref = oracle.attention(Q, K, V, heads, dh)
    ref_base = oracle.attention_ex(Q, K, V, heads, dh, bf16_p=True)
    report("attention numerator, 64-dim heads", M * d, modified=(Os["modified"], ref),
           two_term=(Os["two_term"], ref), baseline=(Os["baseline"], ref))
    assert_bf16_close(Os["modified"], ref)
    assert_bf16_close(Os["baseline"], ref_base)
    n_mod = int(np.count_nonzero(Os["modified"] != ref))
    n_base = int(np.count_nonzero(Os["baseline"] != ref))
    assert n_mod < M * d // 1000, n_mod
    assert n_base > 20 * max(n_mod, 100), (n_base, n_mod)
    assert rel_l2(Os["modified"], ref) < rel_l2(Os["baseline"], ref) / 10
    # weights carried in two BF16 terms (about 17 bits) sit in between
    assert_bf16_close(Os["two_term"], ref)
    assert n_mod <= int(np.count_nonzero(Os["two_term"] != ref)) < n_base
