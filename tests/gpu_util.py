"""Helpers shared by the GPU tests: device buffers, comparisons."""
import os

import numpy as np
import torch

from memory_bounded_weight_amd import psi

MiB = 1 << 20


def dev(a_u16: np.ndarray) -> torch.Tensor:
    """Host bf16 bits -> device int16 tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def empty_bf16(*shape) -> torch.Tensor:
    return torch.empty(*shape, dtype=torch.int16, device="cuda")


def f(u):
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rel_err(got, ref) -> np.ndarray:
    """|g - o| / max(|o|, rms(o)) elementwise (the tolerance metric)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(o ** 2)) if o.size else 1.0
    return np.abs(g - o) / np.maximum(np.abs(o), rms if rms > 0 else 1.0)


def assert_bf16_close(got_bits, ref_bits, tol=2e-2, what="output"):
    r = rel_err(f(got_bits), f(ref_bits))
    diff = int(np.count_nonzero(got_bits != ref_bits))
    assert np.isfinite(f(got_bits)).all(), f"{what}: non-finite values"
    assert r.max() <= tol, f"{what}: max rel {r.max():.3e} > {tol} ({diff} of {got_bits.size} differ)"
    return r.max(), diff


def stream_handle():
    return torch.cuda.current_stream().cuda_stream


def make_arena(arena_bytes, page_bytes, n_pages=2, workspace=0, flags=0):
    """A test arena on torch's current stream.  PSI_TEST_JITTER=1 in the
    environment adds PSI_ARENA_JITTER to every arena (the whole suite then
    runs with pseudo-random delays before each copy and launch; results
    must not change)."""
    if os.environ.get("PSI_TEST_JITTER") == "1" and not flags & psi.PSI_ARENA_SYNC_COPY:
        flags |= psi.PSI_ARENA_JITTER
    d = psi.arena_desc(arena_bytes, page_bytes, n_pages, workspace, 0, stream_handle(), flags)
    return psi.psi_arena_create(d)
