"""CPU oracle of the cache-semantic bucketed hash table.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
library (``hash_table_cache_amd``) never does, and the two share no code.

The arithmetic lives in ``hkv_oracle.cpp`` (plain single-threaded C++,
following Algorithms 1-3 of the HierarchicalKV paper, §3.2-§3.4); this module
only builds it with the host compiler and marshals numpy arrays through ctypes.
Keys, scores, tags and positions are ``numpy.uint64``; values are
``numpy.float32`` rows of ``dim`` elements; found flags are ``numpy.uint8``.
"""

from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
SOURCE = _HERE / "hkv_oracle.cpp"
LIB_PATH = _HERE / "_build" / "liboracle.so"

# Outcome codes written by insert_or_assign (same values as the C enum).
SKIPPED, UPDATED, INSERTED, EVICTED, REJECTED = 0, 1, 2, 3, 4

EMPTY_KEY = np.uint64(0xFFFFFFFFFFFFFFFF)
LOCKED_KEY = np.uint64(0xFFFFFFFFFFFFFFFE)
SLOTS = 128

_lib = None


def build() -> pathlib.Path:
    """Compile the oracle with the host C++ compiler (no GPU code involved)."""
    LIB_PATH.parent.mkdir(parents=True, exist_ok=True)
    tmp = LIB_PATH.with_suffix(".so.tmp")
    subprocess.check_call(
        ["g++", "-O2", "-std=c++17", "-Wall", "-shared", "-fPIC", "-o", str(tmp), str(SOURCE)]
    )
    tmp.replace(LIB_PATH)
    return LIB_PATH


def _u64p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def _f32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _u8p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _u32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def lib():
    """Load the oracle library, building it first if it is not there.
    HKV_ORACLE_LIB names another build of the same source (used by the test
    that plants mistakes in copies of the oracle)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("HKV_ORACLE_LIB")
    if path is None:
        path = LIB_PATH
        if not LIB_PATH.exists():
            build()
    L = ctypes.CDLL(str(path))
    u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
    P64 = ctypes.POINTER(ctypes.c_uint64)
    PF = ctypes.POINTER(ctypes.c_float)
    P8 = ctypes.POINTER(ctypes.c_uint8)
    P32 = ctypes.POINTER(ctypes.c_uint32)
    L.oracle_create.argtypes = [u64, u32, ctypes.c_int, ctypes.c_int]
    L.oracle_create.restype = vp
    L.oracle_destroy.argtypes = [vp]
    L.oracle_destroy.restype = None
    L.oracle_fmix64.argtypes = [u64]
    L.oracle_fmix64.restype = u64
    L.oracle_murmur3_x64_128.argtypes = [vp, u64, u32, P64]
    L.oracle_murmur3_x64_128.restype = None
    L.oracle_route.argtypes = [vp, u64, P64, P64, P64, P8]
    L.oracle_route.restype = None
    L.oracle_route_buckets.argtypes = [u64, ctypes.c_int, u64, P64, P64, P64, P8]
    L.oracle_route_buckets.restype = None
    L.oracle_find.argtypes = [vp, u64, P64, PF, P8, P64, P64]
    L.oracle_find.restype = None
    L.oracle_insert_or_assign.argtypes = [vp, u64, P64, PF, P64, P64, P32]
    L.oracle_insert_or_assign.restype = None
    L.oracle_assign.argtypes = [vp, u64, P64, PF, P64, P64]
    L.oracle_assign.restype = None
    L.oracle_find_pos.argtypes = [vp, u64, P64, P8, P64]
    L.oracle_find_pos.restype = None
    L.oracle_insert_and_evict.argtypes = [vp, u64, P64, PF, P64, P64, P64, PF, P64, P64]
    L.oracle_insert_and_evict.restype = u64
    L.oracle_find_or_insert.argtypes = [vp, u64, P64, PF, P64, P64, P8]
    L.oracle_find_or_insert.restype = None
    L.oracle_size.argtypes = [vp]
    L.oracle_size.restype = u64
    L.oracle_export.argtypes = [vp, u64, u64, P64, PF, P64, P64, P64]
    L.oracle_export.restype = u64
    L.oracle_probe_stats.argtypes = [vp, P64]
    L.oracle_probe_stats.restype = None
    L.oracle_reset_probe_stats.argtypes = [vp]
    L.oracle_reset_probe_stats.restype = None
    _lib = L
    return L


def _keys(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.int64:
        a = a.view(np.uint64)
    if a.dtype != np.uint64:
        raise TypeError(f"keys/scores must be uint64 (or int64 bit patterns), got {a.dtype}")
    return a


def route_buckets(keys, buckets: int, dual: bool = False):
    """(b1, b2, digest) of every key for a table of `buckets` buckets."""
    keys = _keys(keys)
    n = keys.size
    b1 = np.empty(n, np.uint64)
    b2 = np.empty(n, np.uint64)
    d = np.empty(n, np.uint8)
    lib().oracle_route_buckets(int(buckets), int(dual), n, _u64p(keys), _u64p(b1), _u64p(b2), _u8p(d))
    return b1, b2, d


def fmix64(k: int) -> int:
    return int(lib().oracle_fmix64(int(k)))


def murmur3_x64_128(data: bytes, seed: int) -> tuple[int, int]:
    out = np.zeros(2, dtype=np.uint64)
    buf = ctypes.create_string_buffer(bytes(data), max(len(data), 1))
    lib().oracle_murmur3_x64_128(buf, len(data), seed & 0xFFFFFFFF, _u64p(out))
    return int(out[0]), int(out[1])


class OracleTable:
    """Single-threaded CPU table; see ``hkv_oracle.cpp`` for the semantics.

    ``tag_mode=True`` stores one u64 tag per slot instead of ``dim`` floats, so
    that tables whose value rows would not fit in host memory can still be
    followed exactly (the caller derives the row from the tag).
    """

    def __init__(self, capacity: int, dim: int, dual: bool = False, tag_mode: bool = False):
        self._lib = lib()
        self.capacity = int(capacity)
        self.dim = int(dim)
        self.dual = bool(dual)
        self.tag_mode = bool(tag_mode)
        self.buckets = self.capacity // SLOTS
        h = self._lib.oracle_create(self.capacity, self.dim, int(dual), int(tag_mode))
        if not h:
            raise ValueError(f"oracle_create rejected capacity={capacity} dim={dim}")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.oracle_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def route(self, keys):
        keys = _keys(keys)
        n = keys.size
        b1 = np.empty(n, np.uint64)
        b2 = np.empty(n, np.uint64)
        d = np.empty(n, np.uint8)
        self._lib.oracle_route(self._h, n, _u64p(keys), _u64p(b1), _u64p(b2), _u8p(d))
        return b1, b2, d

    def find(self, keys, values_out=None, scores_out=None, tags_out=None):
        """Returns (values, found, scores, tags). Rows/scores/tags of misses keep
        whatever the passed-in output arrays held (zeros if none given)."""
        keys = _keys(keys)
        n = keys.size
        found = np.zeros(n, np.uint8)
        if scores_out is None:
            scores_out = np.zeros(n, np.uint64)
        if self.tag_mode:
            if tags_out is None:
                tags_out = np.zeros(n, np.uint64)
            self._lib.oracle_find(self._h, n, _u64p(keys), None, _u8p(found), _u64p(scores_out), _u64p(tags_out))
            return None, found, scores_out, tags_out
        if values_out is None:
            values_out = np.zeros((n, self.dim), np.float32)
        assert values_out.dtype == np.float32 and values_out.flags.c_contiguous
        self._lib.oracle_find(self._h, n, _u64p(keys), _f32p(values_out), _u8p(found), _u64p(scores_out), None)
        return values_out, found, scores_out, None

    def insert_or_assign(self, keys, scores, values=None, tags=None):
        """Applies the batch in input order; returns one outcome code per key."""
        keys = _keys(keys)
        scores = _keys(scores)
        n = keys.size
        assert scores.size == n
        out = np.zeros(n, np.uint32)
        if self.tag_mode:
            tags = _keys(tags)
            assert tags.size == n
            self._lib.oracle_insert_or_assign(self._h, n, _u64p(keys), None, _u64p(tags), _u64p(scores), _u32p(out))
        else:
            values = np.ascontiguousarray(values, dtype=np.float32)
            assert values.shape == (n, self.dim)
            self._lib.oracle_insert_or_assign(self._h, n, _u64p(keys), _f32p(values), None, _u64p(scores), _u32p(out))
        return out

    def assign(self, keys, values=None, scores=None, tags=None):
        keys = _keys(keys)
        n = keys.size
        if scores is not None:
            scores = _keys(scores)
        if values is not None:
            values = np.ascontiguousarray(values, dtype=np.float32)
            assert values.shape == (n, self.dim)
        if tags is not None:
            tags = _keys(tags)
        self._lib.oracle_assign(self._h, n, _u64p(keys), _f32p(values), _u64p(tags), _u64p(scores))

    def find_pos(self, keys):
        """find* / contains: (found flags, slot positions; 2^64 - 1 on a miss)."""
        keys = _keys(keys)
        n = keys.size
        found = np.zeros(n, np.uint8)
        pos = np.zeros(n, np.uint64)
        self._lib.oracle_find_pos(self._h, n, _u64p(keys), _u8p(found), _u64p(pos))
        return found, pos

    def contains(self, keys) -> np.ndarray:
        return self.find_pos(keys)[0]

    def insert_and_evict(self, keys, scores, values=None, tags=None):
        """Upserts the batch; returns the entries that left or were turned away:
        dict(keys, scores, values | tags), in the order they happened."""
        keys = _keys(keys)
        scores = _keys(scores)
        n = keys.size
        assert scores.size == n
        ek = np.empty(n, np.uint64)
        es = np.empty(n, np.uint64)
        if self.tag_mode:
            tags = _keys(tags)
            et = np.empty(n, np.uint64)
            m = self._lib.oracle_insert_and_evict(self._h, n, _u64p(keys), None, _u64p(tags), _u64p(scores),
                                                  _u64p(ek), None, _u64p(et), _u64p(es))
            return dict(keys=ek[:m], scores=es[:m], tags=et[:m])
        values = np.ascontiguousarray(values, dtype=np.float32)
        assert values.shape == (n, self.dim)
        ev = np.empty((n, self.dim), np.float32)
        m = self._lib.oracle_insert_and_evict(self._h, n, _u64p(keys), _f32p(values), None, _u64p(scores),
                                              _u64p(ek), _f32p(ev), None, _u64p(es))
        return dict(keys=ek[:m], scores=es[:m], values=ev[:m])

    def find_or_insert(self, keys, scores, values=None, tags=None):
        """Returns (rows or tags after the call, found flags). The caller's
        arrays are not modified; copies are returned."""
        keys = _keys(keys)
        scores = _keys(scores)
        n = keys.size
        found = np.zeros(n, np.uint8)
        if self.tag_mode:
            t = np.array(_keys(tags), copy=True)
            self._lib.oracle_find_or_insert(self._h, n, _u64p(keys), None, _u64p(t), _u64p(scores), _u8p(found))
            return t, found
        v = np.array(values, dtype=np.float32, copy=True, order="C")
        assert v.shape == (n, self.dim)
        self._lib.oracle_find_or_insert(self._h, n, _u64p(keys), _f32p(v), None, _u64p(scores), _u8p(found))
        return v, found

    def size(self) -> int:
        return int(self._lib.oracle_size(self._h))

    def export(self, offset: int = 0, n_slots: int | None = None):
        """Occupied slots in [offset, offset + n_slots), ascending position.
        Returns dict(keys, scores, pos, values | tags)."""
        if n_slots is None:
            n_slots = self.capacity - offset
        m_max = max(0, min(n_slots, self.capacity - offset))
        keys = np.empty(m_max, np.uint64)
        scores = np.empty(m_max, np.uint64)
        pos = np.empty(m_max, np.uint64)
        if self.tag_mode:
            tags = np.empty(m_max, np.uint64)
            m = self._lib.oracle_export(self._h, offset, n_slots, _u64p(keys), None, _u64p(scores), _u64p(pos), _u64p(tags))
            return dict(keys=keys[:m], scores=scores[:m], pos=pos[:m], tags=tags[:m])
        values = np.empty((m_max, self.dim), np.float32)
        m = self._lib.oracle_export(self._h, offset, n_slots, _u64p(keys), _f32p(values), _u64p(scores), _u64p(pos), None)
        return dict(keys=keys[:m], scores=scores[:m], pos=pos[:m], values=values[:m])

    def probe_stats(self) -> tuple[int, int]:
        out = np.zeros(2, np.uint64)
        self._lib.oracle_probe_stats(self._h, _u64p(out))
        return int(out[0]), int(out[1])

    def reset_probe_stats(self):
        self._lib.oracle_reset_probe_stats(self._h)
