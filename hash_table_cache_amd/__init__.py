"""Cache-semantic bucketed GPU hash table for MI355X (gfx950).

The table and every operation on it live in the HIP library ``libhkv.so``
behind the C ABI of ``include/hkv.h``; this package is its Python binding.
``HashTable`` owns one table and allocates output tensors; the functions of
``hash_table_cache_amd._native`` mirror the C entry points one to one.
"""

from __future__ import annotations

import torch

from . import _native
from ._native import (  # noqa: F401
    BUCKET_SLOTS,
    EMPTY_KEY,
    HKV_FLAG_RW_LOCK,
    HKV_FLAG_SERIAL_INSERT,
    HKV_FLAG_UNIQUE_KEYS,
    LOCKED_KEY,
    HkvError,
    hkv_assign,
    hkv_contains,
    hkv_create,
    hkv_destroy,
    hkv_export_batch,
    hkv_find,
    hkv_find_or_insert,
    hkv_find_ptr,
    hkv_get_options,
    hkv_insert_and_evict,
    hkv_insert_or_assign,
    hkv_profile_start,
    hkv_profile_stop,
    hkv_set_outcome_counters,
    hkv_size,
)

__all__ = ["HashTable", "HkvError", "BUCKET_SLOTS", "EMPTY_KEY", "LOCKED_KEY", "HKV_FLAG_SERIAL_INSERT",
           "HKV_FLAG_RW_LOCK", "HKV_FLAG_UNIQUE_KEYS"]


class HashTable:
    """One table on one GPU.

    capacity: slots (a multiple of 128); dim: float32 values per row;
    dual_bucket: score-based dual-bucket mode; values_on_host: value rows in
    pinned host memory mapped into the GPU, except the first hbm_value_bytes'
    worth of buckets, which stay in HBM; serial_insert: apply inserts one key
    at a time in input order (deterministic placement, slow); unique_keys:
    the caller guarantees distinct keys in every write batch
    (HKV_FLAG_UNIQUE_KEYS); flags: further HKV_FLAG_* bits
    (HKV_FLAG_RW_LOCK: reader/writer call ordering).
    """

    def __init__(self, capacity: int, dim: int, dual_bucket: bool = False, values_on_host: bool = False,
                 device: int = 0, serial_insert: bool = False, hbm_value_bytes: int = 0, flags: int = 0,
                 unique_keys: bool = False):
        self.capacity = int(capacity)
        self.dim = int(dim)
        self.dual_bucket = bool(dual_bucket)
        self.values_on_host = bool(values_on_host)
        self.device = int(device)
        flags = (int(flags) | (HKV_FLAG_SERIAL_INSERT if serial_insert else 0)
                 | (HKV_FLAG_UNIQUE_KEYS if unique_keys else 0))
        self._outcomes = None
        self._h = hkv_create(capacity, dim, dual_bucket, values_on_host, device, flags, hbm_value_bytes)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            hkv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self):
        return self._h

    def _dev(self):
        return torch.device("cuda", self.device)

    def find(self, keys, values_out=None, found_out=None, scores_out=None, with_scores=False, stream=None):
        n = keys.numel()
        if values_out is None:
            values_out = torch.zeros((n, self.dim), dtype=torch.float32, device=self._dev())
        if found_out is None:
            found_out = torch.empty(n, dtype=torch.uint8, device=self._dev())
        if scores_out is None and with_scores:
            scores_out = torch.zeros(n, dtype=torch.int64, device=self._dev())
        hkv_find(self._h, keys, values_out, found_out, scores_out, stream, dim=self.dim, device=self.device)
        return values_out, found_out, scores_out

    def find_ptr(self, keys, ptrs_out=None, found_out=None, scores_out=None, stream=None):
        """find*: int64 row addresses (0 on a miss) and found flags."""
        n = keys.numel()
        if ptrs_out is None:
            ptrs_out = torch.empty(n, dtype=torch.int64, device=self._dev())
        if found_out is None:
            found_out = torch.empty(n, dtype=torch.uint8, device=self._dev())
        hkv_find_ptr(self._h, keys, ptrs_out, found_out, scores_out, stream, device=self.device)
        return ptrs_out, found_out

    def contains(self, keys, found_out=None, stream=None):
        if found_out is None:
            found_out = torch.empty(keys.numel(), dtype=torch.uint8, device=self._dev())
        hkv_contains(self._h, keys, found_out, stream, device=self.device)
        return found_out

    def insert_or_assign(self, keys, values, scores, stream=None) -> None:
        hkv_insert_or_assign(self._h, keys, values, scores, stream, dim=self.dim, device=self.device)

    def insert_and_evict(self, keys, values, scores, out=None, stream=None):
        """Upserts and returns (keys, values, scores, count) of what was handed
        back; count is a one-element device tensor (nothing synchronizes).
        `out` may pass preallocated (keys, values, scores, count) buffers of
        n entries."""
        n = keys.numel()
        dev = self._dev()
        if out is None:
            out = (torch.empty(max(n, 1), dtype=torch.int64, device=dev),
                   torch.empty((max(n, 1), self.dim), dtype=torch.float32, device=dev),
                   torch.empty(max(n, 1), dtype=torch.int64, device=dev),
                   torch.zeros(1, dtype=torch.int64, device=dev))
        ek, ev, es, cnt = out
        hkv_insert_and_evict(self._h, keys, values, scores, ek, ev, es, cnt, stream, dim=self.dim,
                             device=self.device)
        return ek, ev, es, cnt

    def find_or_insert(self, keys, values, scores, found_out=None, stream=None):
        """values is read and written in place (stored rows of hits)."""
        if found_out is None:
            found_out = torch.empty(keys.numel(), dtype=torch.uint8, device=self._dev())
        hkv_find_or_insert(self._h, keys, values, scores, found_out, stream, dim=self.dim, device=self.device)
        return values, found_out

    def assign(self, keys, values=None, scores=None, stream=None) -> None:
        hkv_assign(self._h, keys, values, scores, stream, dim=self.dim, device=self.device)

    def size(self, stream=None) -> int:
        return hkv_size(self._h, stream, device=self.device)

    OUTCOMES = ("updated", "inserted", "evicted", "rejected")

    def count_outcomes(self, enable: bool = True) -> None:
        """Start (from zero) or stop counting the inserter calls' outcomes."""
        if enable:
            self._outcomes = torch.zeros(4, dtype=torch.int64, device=self._dev())
            torch.cuda.synchronize(self._dev())
            hkv_set_outcome_counters(self._h, self._outcomes)
        else:
            hkv_set_outcome_counters(self._h, None)
            self._outcomes = None

    def outcomes(self) -> dict:
        """{updated, inserted, evicted, rejected} added up since
        count_outcomes(); waits for the device."""
        if self._outcomes is None:
            raise RuntimeError("outcomes are not being counted; call count_outcomes() first")
        torch.cuda.synchronize(self._dev())
        return dict(zip(self.OUTCOMES, (int(v) for v in self._outcomes.cpu().tolist())))

    def profile_start(self) -> None:
        """Time every kernel this table launches from now on (events on its stream)."""
        hkv_profile_start(self._h)

    def profile_stop(self) -> dict:
        """Stop timing; {kernel: (launches, total_ms, max_ms, min_ms, sumsq_ms2, median_ms)}. Waits for the
        timed work."""
        return hkv_profile_stop(self._h)

    def export_batch(self, offset: int = 0, n_slots: int | None = None, with_values: bool = True, stream=None):
        """Returns (keys, values, scores, pos) of the occupied slots in
        [offset, offset + n_slots), in unspecified order; synchronizes."""
        if n_slots is None:
            n_slots = self.capacity - offset
        m = max(0, min(int(n_slots), self.capacity - int(offset)))
        dev = self._dev()
        keys = torch.empty(max(m, 1), dtype=torch.int64, device=dev)
        vals = torch.empty((max(m, 1), self.dim), dtype=torch.float32, device=dev) if with_values else None
        scores = torch.empty(max(m, 1), dtype=torch.int64, device=dev)
        pos = torch.empty(max(m, 1), dtype=torch.int64, device=dev)
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        hkv_export_batch(self._h, offset, n_slots, keys, vals, scores, pos, count, stream,
                         dim=self.dim, device=self.device)
        if stream is not None and not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream), device=dev)
        (stream or torch.cuda.current_stream(dev)).synchronize()
        c = int(count.item())
        return keys[:c], (vals[:c] if vals is not None else None), scores[:c], pos[:c]
