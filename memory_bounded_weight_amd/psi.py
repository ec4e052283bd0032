"""Thin Python binding of the C ABI in ``include/psi.h``.

Argument marshalling only: every step of the paged operator runs in the HIP
library ``libpsi.so`` (built by ``memory_bounded_weight_amd.build``).  The
functions keep the C names and return the C status code, raising
``PsiError`` on failure.  Device pointers and streams are passed as
integers (``tensor.data_ptr()``, ``torch.cuda.current_stream().cuda_stream``);
host page images must be pinned (``torch.empty(..., pin_memory=True)``).

Importing this module loads the library and raises if it has not been
built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PSI_LIB", os.path.join(_HERE, "libpsi.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"HIP library {LIB_PATH} is not built; run "
                      "`python -m memory_bounded_weight_amd.build` (or __graft_entry__.build())")

try:  # bind to the process's HIP runtime (torch's) before loading the library
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------ constants
PSI_OK = 0
PSI_E_INVALID = -1
PSI_E_ARENA_TOO_SMALL = -2
PSI_E_SCRATCH_EXHAUSTED = -3
PSI_E_PAGE_TOO_SMALL = -4
PSI_E_PAGE_BUSY = -5
PSI_E_NOT_PINNED = -6
PSI_E_ALIGN = -7
PSI_E_JOURNAL_KEY = -8
PSI_E_HIP = -9
PSI_E_STATE = -10
PSI_E_JOURNAL_FULL = -11
STATUS_NAMES = {v: k for k, v in dict(globals()).items() if k.startswith("PSI_E_") or k == "PSI_OK"}

PSI_ARENA_SYNC_COPY = 0x1
PSI_ARENA_PROFILE = 0x2
PSI_ARENA_DRY_RUN = 0x4
PSI_ARENA_PROFILE_COPIES = 0x8
PSI_ARENA_JITTER = 0x10

PSI_OP_BASELINE_BIAS = 0x1
PSI_OP_RESIDUAL = 0x2
PSI_OP_STORE_ACC = 0x4
PSI_OP_BF16_SOFTMAX = 0x8
PSI_OP_ATTN_P2 = 0x10
PSI_OP_ATTN_CONFIG_MASK = 0x700


def PSI_OP_ATTN_CONFIG(c):
    """Attention kernel choice in the flags: 0 automatic, 1 128-query, 2
    256-query, 3 lock-step pipelined, 4 ping-pong (all give the same bits)."""
    return (c & 7) << 8


PSI_OP_ATTN_PIPELINED = PSI_OP_ATTN_CONFIG(3)

PSI_ROLE_ATTN_O = 16
PSI_ROLE_FFN_H = 17
PSI_ROLE_FFN_HSTATE = 18
PSI_ROLE_ATTN_OSTATE = 19
PSI_FFN_REUSE = 1
PSI_FFN_RECOMPUTE = 2

PSI_SPLIT_ROWS = 0
PSI_SPLIT_COLS = 1
PSI_SPLIT_TILES = 2
PSI_MAX_PAGES = 8
PSI_JOURNAL_SYNC = 0x1
PSI_JOURNAL_RING = 0x2

_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i = ctypes.c_int
_u = ctypes.c_uint


class psi_arena_desc(ctypes.Structure):
    _fields_ = [("arena_bytes", _sz), ("page_bytes", _sz), ("n_pages", _i),
                ("workspace_bytes", _sz), ("bias_slot_bytes", _sz), ("compute_stream", _vp),
                ("flags", _u)]


class psi_arena_layout(ctypes.Structure):
    _fields_ = [("page_off", _sz * PSI_MAX_PAGES), ("bias_off", _sz * 2),
                ("bias_slot_bytes", _sz), ("workspace_off", _sz), ("scratch_off", _sz),
                ("scratch_bytes", _sz), ("total_bytes", _sz)]


class psi_stats(ctypes.Structure):
    _fields_ = [("arena_bytes", _sz), ("page_bytes", _sz), ("workspace_bytes", _sz),
                ("scratch_bytes", _sz), ("scratch_high_water", _sz),
                ("bytes_h2d", ctypes.c_uint64), ("page_copies", ctypes.c_uint64),
                ("event_waits", ctypes.c_uint64), ("host_syncs", ctypes.c_uint64),
                ("kernel_launches", ctypes.c_uint64),
                ("gemm_ms", ctypes.c_double), ("gemm_launches", ctypes.c_uint64),
                ("gemm_flops", ctypes.c_double),
                ("attn_ms", ctypes.c_double), ("attn_launches", ctypes.c_uint64),
                ("attn_flops", ctypes.c_double),
                ("copy_ms", ctypes.c_double), ("copy_bytes_timed", ctypes.c_uint64),
                ("lent_page_copies", ctypes.c_uint64),
                ("ahead_page_copies", ctypes.c_uint64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class psi_trace_event(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32), ("start_ms", ctypes.c_double),
                ("dur_ms", ctypes.c_double), ("work", ctypes.c_double)]


class psi_matrix(ctypes.Structure):
    _fields_ = [("pages_host", _vp), ("bias_host", _vp), ("rows", _i), ("cols", _i),
                ("split", _i), ("block", _i), ("resident", _i), ("block_cols", _i)]


class psi_block_weights(ctypes.Structure):
    _fields_ = [("Wq", psi_matrix), ("Wk", psi_matrix), ("Wv", psi_matrix), ("Wo", psi_matrix),
                ("U", psi_matrix), ("V", psi_matrix)]


class psi_qk_norm_rope(ctypes.Structure):
    _fields_ = [("gamma_q", _vp), ("gamma_k", _vp), ("eps", ctypes.c_float), ("norm_tile", _i),
                ("cos_q", _vp), ("sin_q", _vp), ("cos_k", _vp), ("sin_k", _vp)]


def qk_norm_rope(gamma_q=None, gamma_k=None, eps=1e-6, norm_tile=0, cos_q=None, sin_q=None,
                 cos_k=None, sin_k=None) -> psi_qk_norm_rope:
    """psi_qk_norm_rope from tensors/arrays/ints (None -> NULL); the
    structure keeps the buffers it points into alive."""
    r = psi_qk_norm_rope(_ptr(gamma_q), _ptr(gamma_k), eps, norm_tile, _ptr(cos_q), _ptr(sin_q),
                         _ptr(cos_k), _ptr(sin_k))
    r._keepalive = (gamma_q, gamma_k, cos_q, sin_q, cos_k, sin_k)
    return r


class psi_key(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("block", ctypes.c_int32),
                ("branch", ctypes.c_int32), ("role", ctypes.c_int32)]


class psi_journal_desc(ctypes.Structure):
    _fields_ = [("ring_slot_bytes", _sz), ("ring_slots", _i), ("store_bytes", _sz), ("flags", _u)]


_P = ctypes.POINTER


def _sig(name, args, res=_i):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_sig("psi_pack_matrix", [_vp, _i, _i, _i, _i, _vp])
_sig("psi_pack_tiles", [_vp, _i, _i, _i, _i, _vp])
_sig("psi_matrix_pages", [_P(psi_matrix)])
_sig("psi_matrix_page_bytes", [_P(psi_matrix), _i], _sz)
_sig("psi_arena_plan", [_P(psi_arena_desc), _P(psi_arena_layout)])
_sig("psi_linear_plan", [_P(psi_arena_desc), _i, _i, _P(psi_matrix), _i, _P(_sz)])
_sig("psi_ffn_plan", [_P(psi_arena_desc), _i, _i, _P(psi_matrix), _P(psi_matrix), _i, _i, _P(_sz)])
_sig("psi_attn_plan", [_P(psi_arena_desc), _i, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                       _P(psi_matrix), _P(psi_matrix), _i, _P(_sz)])
_sig("psi_last_error", [], ctypes.c_char_p)
_sig("psi_version", [], ctypes.c_char_p)
_sig("psi_arena_create", [_P(psi_arena_desc), _P(_vp)])
_sig("psi_arena_destroy", [_vp])
_sig("psi_arena_sync", [_vp])
_sig("psi_arena_set_timing", [_vp, _i])
_sig("psi_arena_stats", [_vp, _P(psi_stats)])
_sig("psi_arena_reset_stats", [_vp])
_sig("psi_arena_trace_start", [_vp, _sz])
_sig("psi_arena_trace_read", [_vp, _P(psi_trace_event), _sz, _P(_sz)])
_sig("psi_arena_device_base", [_vp, _P(_vp), _P(_sz)])
_sig("psi_arena_set_probe", [_vp, _vp, ctypes.c_int32, ctypes.c_int32])
_sig("psi_page_submit", [_vp, _vp, _sz, _P(_i)])
_sig("psi_page_acquire", [_vp, _i, _P(_vp)])
_sig("psi_page_release", [_vp, _i])
_sig("psi_linear_paged", [_vp, _vp, _i, _i, _P(psi_matrix), _vp, _vp, _u])
_sig("psi_linear_resident_noalloc", [_vp, _i, _i, _P(psi_matrix), _vp, _u, _vp])
_sig("psi_ffn_paged", [_vp, _vp, _i, _i, _P(psi_matrix), _P(psi_matrix), _i, _vp, _vp, _u])
_sig("psi_ffn_tiled_plan", [_P(psi_arena_desc), _i, _i, _P(psi_matrix), _P(psi_matrix), _i, _P(_sz)])
_sig("psi_ffn_tiled", [_vp, _vp, _i, _i, _P(psi_matrix), _P(psi_matrix), _i, _vp, ctypes.c_int32,
                       ctypes.c_int32, _vp, _u])
_sig("psi_attn_paged", [_vp, _vp, _i, _vp, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                        _P(psi_matrix), _P(psi_matrix), _vp, _vp, _u])
_sig("psi_attn_ext_plan", [_P(psi_arena_desc), _i, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                           _P(psi_matrix), _P(psi_matrix), _P(psi_qk_norm_rope), _i, _P(_sz)])
_sig("psi_attn_paged_ext", [_vp, _vp, _i, _vp, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                            _P(psi_matrix), _P(psi_matrix), _P(psi_qk_norm_rope), _vp, _vp, _u])
_sig("psi_attn_tiled_plan", [_P(psi_arena_desc), _i, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                             _P(psi_matrix), _P(psi_matrix), _P(_sz)])
_sig("psi_attn_tiled", [_vp, _vp, _i, _vp, _i, _i, _i, _P(psi_matrix), _P(psi_matrix),
                        _P(psi_matrix), _P(psi_matrix), _vp, ctypes.c_int32, ctypes.c_int32, _vp, _u])
_sig("psi_block_lowlive", [_vp, _vp, _i, _i, _i, _P(psi_block_weights), _vp, _u])
_sig("psi_journal_reset", [_vp])
_sig("psi_block_paged", [_vp, _vp, _vp, _i, _i, _i, _P(psi_block_weights), _i, _vp, _vp, _u])
_sig("psi_journal_create", [_P(psi_journal_desc), _P(_vp)])
_sig("psi_journal_destroy", [_vp])
_sig("psi_journal_commit", [_vp, psi_key, _vp, _sz, _vp])
_sig("psi_journal_reload", [_vp, psi_key, _vp, _sz, _vp])
_sig("psi_journal_fence", [_vp, _vp])
_sig("psi_journal_sync", [_vp])
_sig("psi_journal_read", [_vp, psi_key, _vp, _sz])
_sig("psi_journal_counters", [_vp, _P(ctypes.c_uint64), _P(ctypes.c_uint64), _P(ctypes.c_uint64)])

#: every symbol the header declares (checked by the CPU test suite)
EXPORTS = ["psi_pack_matrix", "psi_pack_tiles", "psi_matrix_pages", "psi_matrix_page_bytes", "psi_arena_plan",
           "psi_linear_plan", "psi_ffn_plan", "psi_attn_plan", "psi_last_error", "psi_version",
           "psi_arena_create", "psi_arena_destroy", "psi_arena_sync", "psi_arena_set_timing",
           "psi_arena_stats",
           "psi_arena_reset_stats", "psi_arena_trace_start", "psi_arena_trace_read",
           "psi_arena_device_base", "psi_arena_set_probe", "psi_page_submit",
           "psi_page_acquire", "psi_page_release", "psi_linear_paged",
           "psi_linear_resident_noalloc", "psi_ffn_paged",
           "psi_attn_paged", "psi_block_paged", "psi_ffn_tiled_plan", "psi_ffn_tiled",
           "psi_attn_ext_plan", "psi_attn_paged_ext", "psi_attn_tiled_plan", "psi_attn_tiled",
           "psi_block_lowlive", "psi_journal_reset",
           "psi_journal_create", "psi_journal_destroy",
           "psi_journal_commit", "psi_journal_reload", "psi_journal_fence", "psi_journal_sync",
           "psi_journal_read", "psi_journal_counters"]


class PsiError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        msg = _lib.psi_last_error().decode(errors="replace")
        super().__init__(f"{func} -> {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status, func):
    if status != PSI_OK:
        raise PsiError(status, func)
    return status


def _ptr(t):
    """Device/host address of a torch tensor, numpy array or int (0/None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


# ------------------------------------------------------------- host helpers

def psi_version() -> str:
    return _lib.psi_version().decode()


def psi_last_error() -> str:
    return _lib.psi_last_error().decode(errors="replace")


def psi_pack_matrix(W, rows, cols, split, block, dst):
    return _check(_lib.psi_pack_matrix(_ptr(W), rows, cols, split, block, _ptr(dst)), "psi_pack_matrix")


def psi_pack_tiles(W, rows, cols, block_rows, block_cols, dst):
    return _check(_lib.psi_pack_tiles(_ptr(W), rows, cols, block_rows, block_cols, _ptr(dst)), "psi_pack_tiles")


def make_matrix(pages_host, bias_host, rows, cols, split, block, resident=0, block_cols=0) -> psi_matrix:
    return psi_matrix(_ptr(pages_host), _ptr(bias_host), rows, cols, split, block, int(resident),
                      int(block_cols))


def psi_matrix_pages(m: psi_matrix) -> int:
    return _lib.psi_matrix_pages(ctypes.byref(m))


def psi_matrix_page_bytes(m: psi_matrix, p: int) -> int:
    return _lib.psi_matrix_page_bytes(ctypes.byref(m), p)


def arena_desc(arena_bytes, page_bytes, n_pages=2, workspace_bytes=0, bias_slot_bytes=0,
               compute_stream=None, flags=0) -> psi_arena_desc:
    return psi_arena_desc(arena_bytes, page_bytes, n_pages, workspace_bytes, bias_slot_bytes,
                          compute_stream or None, flags)


def psi_arena_plan(desc: psi_arena_desc) -> psi_arena_layout:
    out = psi_arena_layout()
    _check(_lib.psi_arena_plan(ctypes.byref(desc), ctypes.byref(out)), "psi_arena_plan")
    return out


def _plan_status(st, need):
    return st, need.value


def psi_linear_plan(desc, M, K, W, acc_external=True):
    need = _sz(0)
    st = _lib.psi_linear_plan(ctypes.byref(desc), M, K, ctypes.byref(W), int(acc_external),
                              ctypes.byref(need))
    return _plan_status(st, need)


def psi_ffn_plan(desc, M, d, U, V, token_chunks=1, acc_external=True):
    need = _sz(0)
    st = _lib.psi_ffn_plan(ctypes.byref(desc), M, d, ctypes.byref(U), ctypes.byref(V),
                           token_chunks, int(acc_external), ctypes.byref(need))
    return _plan_status(st, need)


def psi_attn_plan(desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_external=True):
    need = _sz(0)
    st = _lib.psi_attn_plan(ctypes.byref(desc), M, Mc, heads, head_dim, ctypes.byref(Wq),
                            ctypes.byref(Wk), ctypes.byref(Wv), ctypes.byref(Wo),
                            int(acc_external), ctypes.byref(need))
    return _plan_status(st, need)


def psi_attn_ext_plan(desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, nr, acc_external=True):
    need = _sz(0)
    st = _lib.psi_attn_ext_plan(ctypes.byref(desc), M, Mc, heads, head_dim, ctypes.byref(Wq),
                                ctypes.byref(Wk), ctypes.byref(Wv), ctypes.byref(Wo),
                                ctypes.byref(nr) if nr is not None else None, int(acc_external),
                                ctypes.byref(need))
    return _plan_status(st, need)


# -------------------------------------------------------------------- arena

def psi_arena_create(desc: psi_arena_desc) -> int:
    h = _vp()
    _check(_lib.psi_arena_create(ctypes.byref(desc), ctypes.byref(h)), "psi_arena_create")
    return h.value


# Host weight objects (page images, biases, norm parameters) that an
# arena's enqueued operators copy from: the operators return before their
# copies run, and the C ABI requires the host memory to stay valid until
# the compute stream has passed the operator.  The binding keeps the
# Python owners alive until the next psi_arena_sync / psi_arena_destroy,
# so a temporary argument is not freed (and its pinned block handed to
# the next allocation) while a DMA still reads it.
_held: dict = {}


def _hold(arena, *objs):
    h = _held.setdefault(arena, {})
    for o in objs:
        if o is not None:
            h[id(o)] = o


def psi_arena_destroy(arena: int):
    try:
        return _check(_lib.psi_arena_destroy(arena), "psi_arena_destroy")
    finally:
        _held.pop(arena, None)


def psi_arena_sync(arena: int):
    st = _check(_lib.psi_arena_sync(arena), "psi_arena_sync")
    _held.pop(arena, None)
    return st


def psi_arena_set_timing(arena: int, on: bool):
    return _check(_lib.psi_arena_set_timing(arena, int(bool(on))), "psi_arena_set_timing")


def psi_arena_stats(arena: int) -> psi_stats:
    s = psi_stats()
    _check(_lib.psi_arena_stats(arena, ctypes.byref(s)), "psi_arena_stats")
    return s


def psi_arena_reset_stats(arena: int):
    return _check(_lib.psi_arena_reset_stats(arena), "psi_arena_reset_stats")


def psi_arena_trace_start(arena: int, capacity: int = 1 << 16):
    return _check(_lib.psi_arena_trace_start(arena, capacity), "psi_arena_trace_start")


def psi_arena_trace_read(arena: int, capacity: int = 1 << 16):
    """Timeline since psi_arena_trace_start as a list of (kind, start_ms,
    dur_ms, work); kind 0 GEMM, 1 attention, 2 / 3 page copy stream 0 / 1."""
    buf = (psi_trace_event * capacity)()
    n = _sz()
    _check(_lib.psi_arena_trace_read(arena, buf, capacity, ctypes.byref(n)), "psi_arena_trace_read")
    return [(e.kind, e.start_ms, e.dur_ms, e.work) for e in buf[:min(n.value, capacity)]]


def psi_arena_device_base(arena: int):
    b, n = _vp(), _sz()
    _check(_lib.psi_arena_device_base(arena, ctypes.byref(b), ctypes.byref(n)), "psi_arena_device_base")
    return b.value or 0, n.value


def psi_arena_set_probe(arena: int, journal, step: int = 0, block: int = 0):
    return _check(_lib.psi_arena_set_probe(arena, journal or None, step, block), "psi_arena_set_probe")


def psi_page_submit(arena: int, host_pinned, nbytes: int) -> int:
    page = _i(-1)
    _check(_lib.psi_page_submit(arena, _ptr(host_pinned), nbytes, ctypes.byref(page)), "psi_page_submit")
    return page.value


def psi_page_acquire(arena: int, page: int) -> int:
    dev = _vp()
    _check(_lib.psi_page_acquire(arena, page, ctypes.byref(dev)), "psi_page_acquire")
    return dev.value or 0


def psi_page_release(arena: int, page: int):
    return _check(_lib.psi_page_release(arena, page), "psi_page_release")


# ---------------------------------------------------------------- operators

def psi_linear_paged(arena, x, M, K, W: psi_matrix, acc, y, flags=0):
    _hold(arena, W)
    return _check(_lib.psi_linear_paged(arena, _ptr(x), M, K, ctypes.byref(W), _ptr(acc), _ptr(y),
                                        flags), "psi_linear_paged")


PSI_NOALLOC_SCRATCH_BYTES = 16 << 20


def psi_linear_resident_noalloc(x, M, K, W: psi_matrix, y, flags=0, stream=None):
    """Projection over resident pages with no arena and no allocation (the
    K-split accumulator is the library's static per-device array)."""
    return _check(_lib.psi_linear_resident_noalloc(_ptr(x), M, K, ctypes.byref(W), _ptr(y), flags,
                                                   stream), "psi_linear_resident_noalloc")


def psi_ffn_paged(arena, x, M, d, U: psi_matrix, V: psi_matrix, token_chunks, acc, y, flags=0):
    _hold(arena, U, V)
    return _check(_lib.psi_ffn_paged(arena, _ptr(x), M, d, ctypes.byref(U), ctypes.byref(V),
                                     token_chunks, _ptr(acc), _ptr(y), flags), "psi_ffn_paged")


def psi_ffn_tiled_plan(desc, M, d, U: psi_matrix, Vo: psi_matrix, schedule):
    need = _sz(0)
    st = _lib.psi_ffn_tiled_plan(ctypes.byref(desc), M, d, ctypes.byref(U), ctypes.byref(Vo), schedule,
                                 ctypes.byref(need))
    return _plan_status(st, need)


def psi_ffn_tiled(arena, x, M, d, U: psi_matrix, Vo: psi_matrix, schedule, journal, step, block, y, flags=0):
    _hold(arena, U, Vo)
    return _check(_lib.psi_ffn_tiled(arena, _ptr(x), M, d, ctypes.byref(U), ctypes.byref(Vo), schedule,
                                     journal, step, block, _ptr(y), flags), "psi_ffn_tiled")


def psi_attn_paged(arena, x, M, ctx, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc, y, flags=0):
    _hold(arena, Wq, Wk, Wv, Wo)
    return _check(_lib.psi_attn_paged(arena, _ptr(x), M, _ptr(ctx), Mc, heads, head_dim,
                                      ctypes.byref(Wq), ctypes.byref(Wk), ctypes.byref(Wv),
                                      ctypes.byref(Wo), _ptr(acc), _ptr(y), flags), "psi_attn_paged")


def psi_attn_paged_ext(arena, x, M, ctx, Mc, heads, head_dim, Wq, Wk, Wv, Wo, nr, acc, y, flags=0):
    _hold(arena, Wq, Wk, Wv, Wo, nr)
    return _check(_lib.psi_attn_paged_ext(arena, _ptr(x), M, _ptr(ctx), Mc, heads, head_dim,
                                          ctypes.byref(Wq), ctypes.byref(Wk), ctypes.byref(Wv),
                                          ctypes.byref(Wo), ctypes.byref(nr) if nr is not None else None,
                                          _ptr(acc), _ptr(y), flags), "psi_attn_paged_ext")


def psi_attn_tiled_plan(desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo):
    need = _sz(0)
    st = _lib.psi_attn_tiled_plan(ctypes.byref(desc), M, Mc, heads, head_dim, ctypes.byref(Wq),
                                  ctypes.byref(Wk), ctypes.byref(Wv), ctypes.byref(Wo), ctypes.byref(need))
    return _plan_status(st, need)


def psi_attn_tiled(arena, x, M, ctx, Mc, heads, head_dim, Wq, Wk, Wv, Wo, journal, step, block, y, flags=0):
    _hold(arena, Wq, Wk, Wv, Wo)
    return _check(_lib.psi_attn_tiled(arena, _ptr(x), M, _ptr(ctx), Mc, heads, head_dim,
                                      ctypes.byref(Wq), ctypes.byref(Wk), ctypes.byref(Wv),
                                      ctypes.byref(Wo), journal, step, block, _ptr(y), flags),
                  "psi_attn_tiled")


def psi_block_lowlive(arena, x, M, heads, head_dim, w: psi_block_weights, journal, flags=0):
    _hold(arena, w)
    return _check(_lib.psi_block_lowlive(arena, _ptr(x), M, heads, head_dim, ctypes.byref(w), journal,
                                         flags), "psi_block_lowlive")


def psi_journal_reset(j):
    return _check(_lib.psi_journal_reset(j), "psi_journal_reset")


def psi_block_paged(arena, x, x_tmp, M, heads, head_dim, w: psi_block_weights, token_chunks,
                    acc, journal=None, flags=0):
    _hold(arena, w)
    return _check(_lib.psi_block_paged(arena, _ptr(x), _ptr(x_tmp), M, heads, head_dim,
                                       ctypes.byref(w), token_chunks, _ptr(acc), journal or None,
                                       flags), "psi_block_paged")


# ------------------------------------------------------------------ journal

def psi_journal_create(ring_slot_bytes, ring_slots, store_bytes, flags=0) -> int:
    d = psi_journal_desc(ring_slot_bytes, ring_slots, store_bytes, flags)
    h = _vp()
    _check(_lib.psi_journal_create(ctypes.byref(d), ctypes.byref(h)), "psi_journal_create")
    return h.value


def psi_journal_destroy(j):
    return _check(_lib.psi_journal_destroy(j), "psi_journal_destroy")


def key(step=0, block=0, branch=0, role=0) -> psi_key:
    return psi_key(step, block, branch, role)


def psi_journal_commit(j, k: psi_key, dev, nbytes, producer_stream=None):
    return _check(_lib.psi_journal_commit(j, k, _ptr(dev), nbytes, producer_stream or None),
                  "psi_journal_commit")


def psi_journal_reload(j, k: psi_key, dev, nbytes, consumer_stream=None):
    return _check(_lib.psi_journal_reload(j, k, _ptr(dev), nbytes, consumer_stream or None),
                  "psi_journal_reload")


def psi_journal_fence(j, stream=None):
    return _check(_lib.psi_journal_fence(j, stream or None), "psi_journal_fence")


def psi_journal_sync(j):
    return _check(_lib.psi_journal_sync(j), "psi_journal_sync")


def psi_journal_read(j, k: psi_key, host_dst, nbytes):
    return _check(_lib.psi_journal_read(j, k, _ptr(host_dst), nbytes), "psi_journal_read")


def psi_journal_counters(j):
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(_lib.psi_journal_counters(j, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "psi_journal_counters")
    return a.value, b.value, c.value


# ------------------------------------------------------ pinned weight images

def pinned_matrix(W, bias, split, block, block_cols=0) -> psi_matrix:
    """Pack a host bf16 matrix (numpy uint16 [rows, cols]) into a pinned page
    image (torch pinned memory is plumbing only) and describe it as a
    psi_matrix (``block_cols`` for PSI_SPLIT_TILES).  The returned structure
    keeps the pinned buffers alive."""
    import numpy as np
    import torch
    W = np.ascontiguousarray(W, dtype=np.uint16)
    rows, cols = W.shape
    img = torch.empty(rows * cols, dtype=torch.int16, pin_memory=True)
    if split == PSI_SPLIT_TILES:
        psi_pack_tiles(W, rows, cols, block, block_cols, img)
    else:
        psi_pack_matrix(W, rows, cols, split, block, img)
    b = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        assert bias.shape == (rows,)
        b = torch.empty(rows, dtype=torch.int16, pin_memory=True)
        b.copy_(torch.from_numpy(bias.view(np.int16)))
    m = make_matrix(img, b, rows, cols, split, block, 0, block_cols)
    m._keepalive = (img, b)
    return m


def resident_matrix(m: psi_matrix) -> psi_matrix:
    """Device-resident copy of a pinned page image (same packing): the
    operators then consume its pages in place, with no H2D copy."""
    import torch
    img, b = m._keepalive
    dimg = img.to("cuda", non_blocking=False)
    db = b.to("cuda", non_blocking=False) if b is not None else None
    r = make_matrix(dimg, db, m.rows, m.cols, m.split, m.block, 1, m.block_cols)
    r._keepalive = (dimg, db)
    return r


def resident_block_weights(bw: psi_block_weights) -> psi_block_weights:
    """Device-resident copy of a pinned psi_block_weights (same packing)."""
    mats = {n: resident_matrix(m) for n, m in bw._keepalive.items()}
    r = psi_block_weights(mats["Wq"], mats["Wk"], mats["Wv"], mats["Wo"], mats["U"], mats["V"])
    r._keepalive = mats
    return r


def block_weights(w: dict, group_cols: int, hidden_tile: int, resident: bool = False,
                  attn_out_tile: int = 0, ffn_out_tile: int = 0, attn_out_cols: int = 0,
                  ffn_out_cols: int = 0) -> psi_block_weights:
    """psi_block_weights from a dict of host bf16 arrays (Wq..bo, U, a, V, b);
    ``resident`` places the page images in device memory instead.  With
    ``attn_out_tile`` / ``ffn_out_tile`` set, Wo / V are split by rows into
    output tiles of that many rows (the layout psi_block_lowlive takes), and
    with ``attn_out_cols`` / ``ffn_out_cols`` also set into 2-D page tiles of
    that many columns; otherwise by columns (psi_block_paged).  The returned
    structure holds (copies of) the six psi_matrix values and keeps the
    Python objects that own their buffers alive."""
    def out_tiles(W, b, rows, cols):
        if cols:
            return pinned_matrix(W, b, PSI_SPLIT_TILES, rows, cols)
        return pinned_matrix(W, b, PSI_SPLIT_ROWS, rows)

    mats = {n: pinned_matrix(w[n], w["b" + n[1]], PSI_SPLIT_ROWS, group_cols) for n in ("Wq", "Wk", "Wv")}
    mats["Wo"] = (out_tiles(w["Wo"], w["bo"], attn_out_tile, attn_out_cols) if attn_out_tile else
                  pinned_matrix(w["Wo"], w["bo"], PSI_SPLIT_COLS, group_cols))
    mats["U"] = pinned_matrix(w["U"], w["a"], PSI_SPLIT_ROWS, hidden_tile)
    mats["V"] = (out_tiles(w["V"], w["b"], ffn_out_tile, ffn_out_cols) if ffn_out_tile else
                 pinned_matrix(w["V"], w["b"], PSI_SPLIT_COLS, hidden_tile))
    if resident:
        mats = {n: resident_matrix(m) for n, m in mats.items()}
    bw = psi_block_weights(mats["Wq"], mats["Wk"], mats["Wv"], mats["Wo"], mats["U"], mats["V"])
    bw._keepalive = mats
    return bw
