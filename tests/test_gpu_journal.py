"""GPU tests of the host journal: byte-preserving commit/reload in every
transport mode, ordering against producers and consumers, and key errors.

[PSI] sec. II-D ("Precision-Preserving Subtensor Inference for a 22B Joint
Audio-Video Generator under a Fixed GPU Working Set", arXiv 2611.08023):
the D2H copy waits for its producer, reloads keep the previous-consumer
dependencies, and byte-preserving transport preserves outputs.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(scope="module")
def P(psi_lib):
    return psi_lib


@pytest.mark.parametrize("flags", [0, "ring", "sync"])
def test_journal_roundtrip_bytes(P, flags):
    fl = {0: 0, "ring": P.PSI_JOURNAL_RING, "sync": P.PSI_JOURNAL_SYNC}[flags]
    j = P.psi_journal_create(1 * MiB, 3, 64 * MiB, fl)
    try:
        s = torch.cuda.current_stream()
        g = torch.Generator(device="cuda").manual_seed(1)
        sizes = [5 * MiB + 6, 123456, 2 * MiB]
        srcs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda", generator=g) for n in sizes]
        keep = [t.clone() for t in srcs]
        for i, t in enumerate(srcs):
            P.psi_journal_commit(j, P.key(0, i, 0, 1), t, t.numel(), s.cuda_stream)
        # producers' buffers are overwritten after a fence: the journal has the old bytes
        P.psi_journal_fence(j, s.cuda_stream)
        for t in srcs:
            t.zero_()
        outs = [torch.empty_like(t) for t in srcs]
        for i, o in enumerate(outs):
            P.psi_journal_reload(j, P.key(0, i, 0, 1), o, o.numel(), s.cuda_stream)
        torch.cuda.synchronize()
        for o, k in zip(outs, keep):
            assert torch.equal(o, k)
        host = np.empty(sizes[1], np.uint8)
        P.psi_journal_read(j, P.key(0, 1, 0, 1), host, sizes[1])
        assert np.array_equal(host, keep[1].cpu().numpy())
        d2h, h2d, n = P.psi_journal_counters(j)
        assert n == 3 and d2h == sum(sizes) and h2d == sum(sizes)
    finally:
        P.psi_journal_destroy(j)


def test_journal_key_errors(P):
    j = P.psi_journal_create(1 * MiB, 2, 4 * MiB, 0)
    try:
        t = torch.ones(1024, dtype=torch.uint8, device="cuda")
        P.psi_journal_commit(j, P.key(1, 2, 3, 4), t, 1024)
        with pytest.raises(P.PsiError) as e:
            P.psi_journal_commit(j, P.key(1, 2, 3, 4), t, 1024)
        assert e.value.status == P.PSI_E_JOURNAL_KEY
        with pytest.raises(P.PsiError) as e:
            P.psi_journal_reload(j, P.key(9, 9, 9, 9), t, 1024)
        assert e.value.status == P.PSI_E_JOURNAL_KEY
        with pytest.raises(P.PsiError) as e:
            P.psi_journal_reload(j, P.key(1, 2, 3, 4), t, 512)
        assert e.value.status == P.PSI_E_JOURNAL_KEY
        big = torch.ones(8 * MiB, dtype=torch.uint8, device="cuda")
        with pytest.raises(P.PsiError) as e:
            P.psi_journal_commit(j, P.key(2, 0, 0, 0), big, big.numel())
        assert e.value.status == P.PSI_E_JOURNAL_FULL
        P.psi_journal_sync(j)
    finally:
        P.psi_journal_destroy(j)


def test_journal_commit_follows_producer(P):
    """A commit enqueued right after a producer kernel sees the producer's
    final bytes (the D2H copy waits for the producer)."""
    j = P.psi_journal_create(1 * MiB, 2, 64 * MiB, 0)
    try:
        s = torch.cuda.current_stream()
        x = torch.zeros(4 * MiB, dtype=torch.int32, device="cuda")
        for step in range(3):
            P.psi_journal_fence(j, s.cuda_stream)  # the overwrite follows earlier commits
            x.add_(step + 1)  # producer on the compute stream
            P.psi_journal_commit(j, P.key(step), x, x.numel() * 4, s.cuda_stream)
        P.psi_journal_sync(j)
        expect = 0
        for step in range(3):
            expect += step + 1
            out = np.empty(4 * MiB, np.int32)
            P.psi_journal_read(j, P.key(step), out, out.nbytes)
            assert (out == expect).all()
    finally:
        P.psi_journal_destroy(j)


@pytest.mark.parametrize("flags", [0, "ring"])
def test_journal_reset_reuses_store_in_stream_order(P, flags):
    """psi_journal_reset drops every key and reuses the store from its
    start without a host wait: a reload enqueued before the reset still
    reads the old bytes, a commit after it writes the same store bytes."""
    fl = {0: 0, "ring": P.PSI_JOURNAL_RING}[flags]
    n = 3 * MiB
    j = P.psi_journal_create(1 * MiB, 4, n + MiB, fl)  # room for one entry only
    try:
        s = torch.cuda.current_stream().cuda_stream
        a = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        b = torch.full((n,), 9, dtype=torch.uint8, device="cuda")
        out_a = torch.empty_like(a)
        out_b = torch.empty_like(b)
        P.psi_journal_commit(j, P.key(0, 0, 0, 1), a, n, s)
        P.psi_journal_reload(j, P.key(0, 0, 0, 1), out_a, n, s)
        with pytest.raises(P.PsiError) as e:  # the store is full
            P.psi_journal_commit(j, P.key(0, 0, 1, 1), b, n, s)
        assert e.value.status == P.PSI_E_JOURNAL_FULL
        P.psi_journal_reset(j)
        with pytest.raises(P.PsiError) as e:
            P.psi_journal_reload(j, P.key(0, 0, 0, 1), out_b, n, s)
        assert e.value.status == P.PSI_E_JOURNAL_KEY
        P.psi_journal_commit(j, P.key(0, 0, 0, 1), b, n, s)  # same key, same store bytes
        P.psi_journal_reload(j, P.key(0, 0, 0, 1), out_b, n, s)
        torch.cuda.synchronize()
        P.psi_journal_sync(j)
        assert torch.equal(out_a, a) and torch.equal(out_b, b)
        assert P.psi_journal_counters(j) == (2 * n, 2 * n, 1)
    finally:
        P.psi_journal_destroy(j)
