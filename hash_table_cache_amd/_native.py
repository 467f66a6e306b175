"""ctypes binding of ``libhkv.so`` (the C ABI of ``include/hkv.h``).

Argument marshalling only: every step of every operation runs in the HIP
library. Tensors are passed by ``data_ptr()``; the stream defaults to torch's
current stream on the table's device. The library is loaded on first use
(``load()``), so that the build script can run from a fresh checkout; if it
has not been built by then, the call raises ImportError. There is no
fallback implementation.

64-bit keys and scores are ``torch.int64`` (or ``torch.uint64``) tensors that
hold the unsigned bit patterns.
"""

from __future__ import annotations

import ctypes
import pathlib

import torch

LIB_PATH = pathlib.Path(__file__).resolve().parent / "_lib" / "libhkv.so"

HKV_OK = 0
HKV_EINVAL = -1
HKV_ENOMEM = -2
HKV_EHIP = -3
HKV_EUNSUPPORTED = -4
HKV_FLAG_SERIAL_INSERT = 0x1
HKV_FLAG_RW_LOCK = 0x2
HKV_FLAG_UNIQUE_KEYS = 0x4
NOALLOC_MAX_KEYS = 1 << 21
BUCKET_SLOTS = 128
EMPTY_KEY = 0xFFFFFFFFFFFFFFFF
LOCKED_KEY = 0xFFFFFFFFFFFFFFFE

# Every entry point declared in include/hkv.h.
EXPORTS = (
    "hkv_create",
    "hkv_destroy",
    "hkv_get_options",
    "hkv_find",
    "hkv_find_ptr",
    "hkv_contains",
    "hkv_insert_or_assign",
    "hkv_insert_or_assign_noalloc",
    "hkv_insert_and_evict",
    "hkv_find_or_insert",
    "hkv_assign",
    "hkv_size",
    "hkv_export_batch",
    "hkv_set_outcome_counters",
    "hkv_profile_start",
    "hkv_profile_stop",
    "hkv_last_error",
)


class HkvOptions(ctypes.Structure):
    _fields_ = [
        ("capacity", ctypes.c_uint64),
        ("dim", ctypes.c_uint32),
        ("bucket_slots", ctypes.c_uint32),
        ("dual_bucket", ctypes.c_uint32),
        ("values_on_host", ctypes.c_uint32),
        ("device", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("hbm_value_bytes", ctypes.c_uint64),
    ]


class HkvKernelStat(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 32),
        ("launches", ctypes.c_uint64),
        ("total_ms", ctypes.c_double),
        ("max_ms", ctypes.c_double),
        ("min_ms", ctypes.c_double),
        ("sumsq_ms2", ctypes.c_double),
        ("median_ms", ctypes.c_double),
    ]


class HkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hkv status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python -m hash_table_cache_amd.build`"
        )
    L = ctypes.CDLL(str(LIB_PATH))
    vp, u64, st = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32
    L.hkv_create.argtypes = [ctypes.POINTER(HkvOptions), ctypes.POINTER(ctypes.c_void_p)]
    L.hkv_create.restype = st
    L.hkv_destroy.argtypes = [vp]
    L.hkv_destroy.restype = st
    L.hkv_get_options.argtypes = [vp, ctypes.POINTER(HkvOptions)]
    L.hkv_get_options.restype = st
    L.hkv_find.argtypes = [vp, u64, vp, vp, vp, vp, vp]
    L.hkv_find.restype = st
    L.hkv_find_ptr.argtypes = [vp, u64, vp, vp, vp, vp, vp]
    L.hkv_find_ptr.restype = st
    L.hkv_contains.argtypes = [vp, u64, vp, vp, vp]
    L.hkv_contains.restype = st
    L.hkv_insert_or_assign.argtypes = [vp, u64, vp, vp, vp, vp]
    L.hkv_insert_or_assign.restype = st
    L.hkv_insert_or_assign_noalloc.argtypes = [vp, u64, vp, vp, vp, vp]
    L.hkv_insert_or_assign_noalloc.restype = st
    L.hkv_insert_and_evict.argtypes = [vp, u64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.hkv_insert_and_evict.restype = st
    L.hkv_find_or_insert.argtypes = [vp, u64, vp, vp, vp, vp, vp]
    L.hkv_find_or_insert.restype = st
    L.hkv_assign.argtypes = [vp, u64, vp, vp, vp, vp]
    L.hkv_assign.restype = st
    L.hkv_size.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64), vp]
    L.hkv_size.restype = st
    L.hkv_export_batch.argtypes = [vp, u64, u64, vp, vp, vp, vp, vp, vp]
    L.hkv_export_batch.restype = st
    L.hkv_set_outcome_counters.argtypes = [vp, vp]
    L.hkv_set_outcome_counters.restype = st
    L.hkv_profile_start.argtypes = [vp]
    L.hkv_profile_start.restype = st
    L.hkv_profile_stop.argtypes = [vp, ctypes.POINTER(HkvKernelStat), ctypes.c_uint32,
                                   ctypes.POINTER(ctypes.c_uint32)]
    L.hkv_profile_stop.restype = st
    L.hkv_last_error.argtypes = []
    L.hkv_last_error.restype = ctypes.c_char_p
    return L


_LIB = None


def load() -> ctypes.CDLL:
    """The loaded ``libhkv.so`` (loaded on the first call)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def _check(status: int) -> None:
    if status != HKV_OK:
        raise HkvError(status, load().hkv_last_error().decode(errors="replace"))


_U64_DTYPES = (torch.int64, torch.uint64)


def _ptr(t, dtypes, numel, name, nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr() if t.numel() else None


def _stream(stream, device: int):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def hkv_create(capacity: int, dim: int, dual_bucket: bool = False, values_on_host: bool = False,
               device: int = 0, flags: int = 0, hbm_value_bytes: int = 0) -> ctypes.c_void_p:
    opt = HkvOptions(int(capacity), int(dim), BUCKET_SLOTS, int(bool(dual_bucket)),
                     int(bool(values_on_host)), int(device), int(flags), int(hbm_value_bytes))
    h = ctypes.c_void_p()
    _check(load().hkv_create(ctypes.byref(opt), ctypes.byref(h)))
    return h


def hkv_destroy(table) -> None:
    _check(load().hkv_destroy(table))


def hkv_get_options(table) -> HkvOptions:
    o = HkvOptions()
    _check(load().hkv_get_options(table, ctypes.byref(o)))
    return o


def hkv_find(table, keys, values_out, found_out, scores_out=None, stream=None, *, dim, device):
    n = keys.numel()
    _check(load().hkv_find(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values_out, (torch.float32,), n * dim, "values_out"),
        _ptr(found_out, (torch.uint8, torch.bool), n, "found_out"),
        _ptr(scores_out, _U64_DTYPES, n, "scores_out", nullable=True),
        _stream(stream, device)))


def hkv_find_ptr(table, keys, ptrs_out, found_out=None, scores_out=None, stream=None, *, device):
    """ptrs_out: int64 tensor of n row addresses (0 on a miss)."""
    n = keys.numel()
    _check(load().hkv_find_ptr(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(ptrs_out, _U64_DTYPES, n, "ptrs_out"),
        _ptr(found_out, (torch.uint8, torch.bool), n, "found_out", nullable=True),
        _ptr(scores_out, _U64_DTYPES, n, "scores_out", nullable=True),
        _stream(stream, device)))


def hkv_contains(table, keys, found_out, stream=None, *, device):
    n = keys.numel()
    _check(load().hkv_contains(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(found_out, (torch.uint8, torch.bool), n, "found_out"),
        _stream(stream, device)))


def hkv_insert_and_evict(table, keys, values, scores, ev_keys, ev_values, ev_scores, ev_count, stream=None, *,
                         dim, device):
    n = keys.numel()
    _check(load().hkv_insert_and_evict(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values, (torch.float32,), n * dim, "values"),
        _ptr(scores, _U64_DTYPES, n, "scores"),
        _ptr(ev_keys, _U64_DTYPES, n, "evicted_keys"),
        _ptr(ev_values, (torch.float32,), n * dim, "evicted_values", nullable=True),
        _ptr(ev_scores, _U64_DTYPES, n, "evicted_scores", nullable=True),
        _ptr(ev_count, _U64_DTYPES, 1, "evicted_count"),
        _stream(stream, device)))


def hkv_find_or_insert(table, keys, values, scores, found_out=None, stream=None, *, dim, device):
    n = keys.numel()
    _check(load().hkv_find_or_insert(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values, (torch.float32,), n * dim, "values"),
        _ptr(scores, _U64_DTYPES, n, "scores"),
        _ptr(found_out, (torch.uint8, torch.bool), n, "found_out", nullable=True),
        _stream(stream, device)))


def hkv_insert_or_assign(table, keys, values, scores, stream=None, *, dim, device):
    n = keys.numel()
    _check(load().hkv_insert_or_assign(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values, (torch.float32,), n * dim, "values"),
        _ptr(scores, _U64_DTYPES, n, "scores"),
        _stream(stream, device)))


def hkv_insert_or_assign_noalloc(table, keys, values, scores, stream=None, *, dim, device):
    n = keys.numel()
    _check(load().hkv_insert_or_assign_noalloc(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values, (torch.float32,), n * dim, "values"),
        _ptr(scores, _U64_DTYPES, n, "scores"),
        _stream(stream, device)))


def hkv_assign(table, keys, values=None, scores=None, stream=None, *, dim, device):
    n = keys.numel()
    _check(load().hkv_assign(
        table, n,
        _ptr(keys, _U64_DTYPES, n, "keys"),
        _ptr(values, (torch.float32,), n * dim, "values", nullable=True),
        _ptr(scores, _U64_DTYPES, n, "scores", nullable=True),
        _stream(stream, device)))


def hkv_size(table, stream=None, *, device) -> int:
    out = ctypes.c_uint64(0)
    _check(load().hkv_size(table, ctypes.byref(out), _stream(stream, device)))
    return int(out.value)


def hkv_export_batch(table, offset, n_slots, keys_out, values_out, scores_out, pos_out, count_out,
                     stream=None, *, dim, device):
    m = int(n_slots)
    _check(load().hkv_export_batch(
        table, int(offset), m,
        _ptr(keys_out, _U64_DTYPES, 0, "keys_out"),
        _ptr(values_out, (torch.float32,), 0, "values_out", nullable=True),
        _ptr(scores_out, _U64_DTYPES, 0, "scores_out", nullable=True),
        _ptr(pos_out, _U64_DTYPES, 0, "pos_out", nullable=True),
        _ptr(count_out, _U64_DTYPES, 1, "count_out"),
        _stream(stream, device)))


def hkv_set_outcome_counters(table, counts) -> None:
    """counts: a device tensor of 4 int64 (updated, inserted, evicted,
    rejected) that the inserter calls add to, or None to stop counting."""
    _check(load().hkv_set_outcome_counters(table, _ptr(counts, _U64_DTYPES, 4, "counts", nullable=True)))


def hkv_profile_start(table) -> None:
    _check(load().hkv_profile_start(table))


def hkv_profile_stop(table) -> dict:
    """Returns {kernel name: (launches, total_ms, max_ms, min_ms, sumsq_ms2, median_ms)}."""
    cap = 16
    out = (HkvKernelStat * cap)()
    count = ctypes.c_uint32(0)
    _check(load().hkv_profile_stop(table, out, cap, ctypes.byref(count)))
    return {out[j].name.decode(): (int(out[j].launches), float(out[j].total_ms), float(out[j].max_ms),
                                   float(out[j].min_ms), float(out[j].sumsq_ms2), float(out[j].median_ms))
            for j in range(min(cap, count.value))}
