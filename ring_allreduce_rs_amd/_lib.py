"""ctypes binding of libar.so -- argument marshalling only.

Every reduction runs in the HIP kernels behind the C ABI (include/ar.h).  If
the library is missing this module raises at import: there is no CPU
fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libar.so")

AR_MAX_RANKS = 64
AR_GRAPHS_MAX_BYTES_DEFAULT = 8 << 20

AR_OK = 0
AR_ERR_INVALID_ARG = 1
AR_ERR_UNSUPPORTED = 2
AR_ERR_RUNTIME = 3
AR_ERR_NO_MEMORY = 4

DTYPES = {"int32": 0, "float32": 1, "bfloat16": 2}
OPS = {"sum": 0, "max": 1, "avg": 2}
ALGOS = {"ring_step": 0, "ring_fused": 1, "tree": 2, "halving_doubling": 3, "auto": 4,
         "double_tree": 5, "tree_fused": 6, "halving_doubling_fused": 7, "double_tree_fused": 8}
ALGO_NAMES = {v: k for k, v in ALGOS.items()}

# every symbol include/ar.h declares
EXPORTS = (
    "ar_create", "ar_set_stream", "ar_set_graphs", "ar_set_pointer_cache",
    "ar_set_residency_caps", "ar_residency_probe", "ar_allreduce",
    "ar_reduce_scatter", "ar_allgather", "ar_ring_rs_step", "ar_ring_ag_step", "ar_tree_step",
    "ar_hd_rs_step", "ar_hd_ag_step", "ar_dtree_step", "ar_chunk_range", "ar_predict_us",
    "ar_auto_algo", "ar_copy", "ar_stream", "ar_stream_timeline", "ar_check", "ar_check_noalloc",
    "ar_status_string",
    "ar_last_error", "ar_destroy",
)


class ArError(RuntimeError):
    """A non-AR_OK status from the C ABI."""

    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.func = func
        self.detail = detail
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading torch
    # first makes libar.so bind to that same runtime instead of pulling in a
    # second one from /opt/rocm, which would fail to open the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python ring_allreduce_rs_amd/_build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i, cp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_char_p
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "ar_create": ([ctypes.POINTER(vp), i, vp], i),
        "ar_set_stream": ([vp, vp], i),
        "ar_set_graphs": ([vp, sz], i),
        "ar_set_pointer_cache": ([vp, i], i),
        "ar_set_residency_caps": ([vp, i], i),
        "ar_residency_probe": ([vp, ctypes.c_uint, ctypes.c_uint, ctypes.POINTER(ctypes.c_uint),
                                ctypes.POINTER(ctypes.c_uint), ctypes.POINTER(ctypes.c_uint)], i),
        "ar_allreduce": ([vp, pp, i, sz, i, i, i], i),
        "ar_reduce_scatter": ([vp, pp, i, sz, i, i, i], i),
        "ar_allgather": ([vp, pp, i, sz, i, i], i),
        "ar_ring_rs_step": ([vp, pp, i, sz, i, i, i], i),
        "ar_ring_ag_step": ([vp, pp, i, sz, i, i], i),
        "ar_tree_step": ([vp, pp, i, sz, i, i, i], i),
        "ar_hd_rs_step": ([vp, pp, i, sz, i, i, i], i),
        "ar_hd_ag_step": ([vp, pp, i, sz, i, i], i),
        "ar_dtree_step": ([vp, pp, i, sz, i, i, i], i),
        "ar_chunk_range": ([sz, i, i, ctypes.POINTER(sz), ctypes.POINTER(sz)], i),
        "ar_predict_us": ([i, i, sz, i, ctypes.POINTER(ctypes.c_double)], i),
        "ar_auto_algo": ([i, sz, i, ctypes.POINTER(i)], i),
        "ar_copy": ([vp, vp, vp, sz], i),
        "ar_stream": ([vp, pp, i, pp, i, sz], i),
        "ar_stream_timeline": ([vp, pp, i, sz, ctypes.c_uint, vp, sz, ctypes.POINTER(sz),
                                ctypes.POINTER(ctypes.c_uint)], i),
        "ar_check": ([vp, pp, i, sz, i, vp, vp, vp], i),
        "ar_check_noalloc": ([vp, pp, i, sz, i, vp, vp, vp], i),
        "ar_status_string": ([i], cp),
        "ar_last_error": ([vp], cp),
        "ar_destroy": ([vp], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()

# The same library's entry points without argtypes, for pre-bound calls whose
# arguments are converted to ctypes objects once: a call then skips the
# per-argument conversion checks (about half of a binding call's host time).
_raw = ctypes.CDLL(LIB_PATH)


def raw_fn(name: str):
    fn = getattr(_raw, name)
    fn.restype = ctypes.c_int
    return fn


def _status_name(s: int) -> str:
    return lib.ar_status_string(s).decode()


def chunk_range(count: int, nranks: int, chunk: int) -> tuple[int, int]:
    """(offset, length) of chunk ``chunk`` -- host-only, no GPU needed."""
    off, ln = ctypes.c_size_t(), ctypes.c_size_t()
    st = lib.ar_chunk_range(count, nranks, chunk, ctypes.byref(off), ctypes.byref(ln))
    if st != AR_OK:
        raise ArError(st, "ar_chunk_range", f"count={count} nranks={nranks} chunk={chunk}")
    return off.value, ln.value


def predict_us(algo: str, nranks: int, count: int, dtype: str) -> float:
    """The library's alpha-beta model time for one AllReduce (host-only)."""
    out = ctypes.c_double()
    st = lib.ar_predict_us(ALGOS[algo], nranks, count, DTYPES[dtype], ctypes.byref(out))
    if st != AR_OK:
        raise ArError(st, "ar_predict_us", f"{algo} nranks={nranks} count={count}")
    return out.value


def auto_algo(nranks: int, count: int, dtype: str) -> str:
    """The algorithm AR_ALGO_AUTO picks for this AllReduce shape (host-only)."""
    out = ctypes.c_int()
    st = lib.ar_auto_algo(nranks, count, DTYPES[dtype], ctypes.byref(out))
    if st != AR_OK:
        raise ArError(st, "ar_auto_algo", f"nranks={nranks} count={count}")
    return ALGO_NAMES[out.value]


class Context:
    """An ar_ctx bound to one device and a HIP stream (a raw hipStream_t int)."""

    def __init__(self, device: int = 0, stream: int | None = None):
        h = ctypes.c_void_p()
        st = lib.ar_create(ctypes.byref(h), device, stream or None)
        if st != AR_OK:
            raise ArError(st, "ar_create", lib.ar_last_error(None).decode())
        self._h = h
        self.device = device
        self._stream = stream or 0
        # the torch wrappers derive every count from the tensors themselves,
        # so a cached pointer set can never be used with more bytes than its
        # allocations now hold
        self._check(lib.ar_set_pointer_cache(self._h, 1), "ar_set_pointer_cache")

    @property
    def handle(self):
        return self._h

    def set_stream(self, stream: int | None) -> None:
        s = stream or 0
        if s != self._stream:
            self._check(lib.ar_set_stream(self._h, s or None), "ar_set_stream")
            self._stream = s

    def set_graphs(self, max_bytes_per_rank: int) -> None:
        """Replay multi-launch collectives of at most this many bytes per rank
        from recorded HIP graphs; 0 turns replay off (ar_set_graphs)."""
        self._check(lib.ar_set_graphs(self._h, max_bytes_per_rank), "ar_set_graphs")

    def residency_probe(self, lds_bytes: int, blocks: int = 256 * 40) -> dict:
        """The most one-wave blocks a compute unit held at once under an LDS
        reservation of lds_bytes (ar_residency_probe): the largest and the
        smallest per-CU maximum and the number of CUs that ran a block."""
        hi, lo, n = ctypes.c_uint(), ctypes.c_uint(), ctypes.c_uint()
        self._check(lib.ar_residency_probe(self._h, lds_bytes, blocks, ctypes.byref(hi),
                                           ctypes.byref(lo), ctypes.byref(n)),
                    "ar_residency_probe")
        return {"max_per_cu": hi.value, "min_per_cu": lo.value, "cus": n.value}

    def set_residency_caps(self, enable: bool) -> None:
        """Residency caps of the large one-pass calls on (the default) or off
        (ar_set_residency_caps); results are the same bits either way."""
        self._check(lib.ar_set_residency_caps(self._h, 1 if enable else 0),
                    "ar_set_residency_caps")

    def last_error(self) -> str:
        return lib.ar_last_error(self._h).decode()

    def _check(self, st: int, func: str) -> None:
        if st != AR_OK:
            raise ArError(st, func, self.last_error())

    # raw-pointer entry points (same names and arguments as the C ABI)
    def allreduce_ptrs(self, ptrs, count, dtype, op, algo):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_allreduce(self._h, arr, len(ptrs), count, DTYPES[dtype], OPS[op],
                                     ALGOS[algo]), "ar_allreduce")

    def reduce_scatter_ptrs(self, ptrs, count, dtype, op, algo):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_reduce_scatter(self._h, arr, len(ptrs), count, DTYPES[dtype],
                                          OPS[op], ALGOS[algo]), "ar_reduce_scatter")

    def allgather_ptrs(self, ptrs, count, dtype, algo):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_allgather(self._h, arr, len(ptrs), count, DTYPES[dtype],
                                     ALGOS[algo]), "ar_allgather")

    def ring_rs_step_ptrs(self, ptrs, count, dtype, op, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_ring_rs_step(self._h, arr, len(ptrs), count, DTYPES[dtype],
                                        OPS[op], step), "ar_ring_rs_step")

    def ring_ag_step_ptrs(self, ptrs, count, dtype, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_ring_ag_step(self._h, arr, len(ptrs), count, DTYPES[dtype], step),
                    "ar_ring_ag_step")

    def tree_step_ptrs(self, ptrs, count, dtype, op, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_tree_step(self._h, arr, len(ptrs), count, DTYPES[dtype], OPS[op],
                                     step), "ar_tree_step")

    def hd_rs_step_ptrs(self, ptrs, count, dtype, op, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_hd_rs_step(self._h, arr, len(ptrs), count, DTYPES[dtype], OPS[op],
                                      step), "ar_hd_rs_step")

    def hd_ag_step_ptrs(self, ptrs, count, dtype, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_hd_ag_step(self._h, arr, len(ptrs), count, DTYPES[dtype], step),
                    "ar_hd_ag_step")

    def dtree_step_ptrs(self, ptrs, count, dtype, op, step):
        arr = _ptr_array(ptrs)
        self._check(lib.ar_dtree_step(self._h, arr, len(ptrs), count, DTYPES[dtype], OPS[op],
                                      step), "ar_dtree_step")

    def copy_ptrs(self, dst, src, nbytes):
        self._check(lib.ar_copy(self._h, dst, src, nbytes), "ar_copy")

    def check_ptrs(self, ptrs, count, dtype, ref, bound, result):
        self._check(lib.ar_check(self._h, _ptr_array(ptrs), len(ptrs), count, DTYPES[dtype],
                                 ref or None, bound or None, result or None), "ar_check")

    def check_noalloc_ptrs(self, ptrs, count, dtype, ref, bound, result):
        self._check(lib.ar_check_noalloc(self._h, _ptr_array(ptrs), len(ptrs), count,
                                         DTYPES[dtype], ref or None, bound or None,
                                         result or None), "ar_check_noalloc")

    def stream_ptrs(self, srcs, dsts, nbytes):
        self._check(lib.ar_stream(self._h, _ptr_array(srcs), len(srcs), _ptr_array(dsts),
                                  len(dsts), nbytes), "ar_stream")

    def stream_timeline_ptrs(self, ptrs, nbytes, lds_bytes, ts_ptr, ts_len):
        """ar_stream_timeline: returns (blocks, wall-clock kHz)."""
        blocks, khz = ctypes.c_size_t(), ctypes.c_uint()
        self._check(lib.ar_stream_timeline(self._h, _ptr_array(ptrs), len(ptrs), nbytes,
                                           lds_bytes, ts_ptr, ts_len, ctypes.byref(blocks),
                                           ctypes.byref(khz)), "ar_stream_timeline")
        return blocks.value, khz.value

    def close(self) -> None:
        if self._h:
            lib.ar_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr_array(ptrs):
    n = len(ptrs)
    return (ctypes.c_void_p * max(n, 1))(*ptrs)
