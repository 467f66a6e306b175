"""Test-side models and comparisons.

``TopKModel`` is the plain definition of what a single-bucket table holds
(the closed form that the bucket-local eviction and admission of §3.3,
Algorithm 2, reach when scores never decrease): bucket b holds the
min(128, m_b) highest entries by (latest score, key) among the m_b distinct
keys ever routed to b by insert_or_assign, each with the value and score of its
last write. It knows nothing about slots, digests, eviction order or the
oracle's code; bucket routing is taken from the oracle's ``route`` (pinned on
its own through the SMHasher check of fmix64).
"""

from __future__ import annotations

import numpy as np

SLOTS = 128


def as_u64(a) -> np.ndarray:
    if not isinstance(a, np.ndarray):
        return np.array([int(x) for x in a], dtype=np.uint64)
    a = np.ascontiguousarray(a)
    if a.dtype == np.int64:
        return a.view(np.uint64)
    return a.astype(np.uint64)


class TopKModel:
    def __init__(self, route_fn, dim: int | None = None):
        self.route = route_fn  # keys (u64 array) -> buckets (u64 array)
        self.dim = dim
        self.score = {}
        self.payload = {}
        self.bucket = {}

    def insert_or_assign(self, keys, scores, payload):
        keys = as_u64(keys)
        scores = as_u64(scores)
        buckets = self.route(keys)
        for i, k in enumerate(keys.tolist()):
            self.score[k] = int(scores[i])
            self.payload[k] = payload[i]
            self.bucket[k] = int(buckets[i])

    def assign(self, keys, scores=None, payload=None):
        res = self.resident_keys()
        keys = as_u64(keys)
        for i, k in enumerate(keys.tolist()):
            if k not in res:
                continue
            if scores is not None:
                self.score[k] = int(as_u64(scores)[i])
            if payload is not None:
                self.payload[k] = payload[i]

    def _arrays(self):
        ks = np.fromiter(self.score.keys(), dtype=np.uint64, count=len(self.score))
        sc = np.fromiter((self.score[k] for k in self.score), dtype=np.uint64, count=len(self.score))
        bk = np.fromiter((self.bucket[k] for k in self.score), dtype=np.uint64, count=len(self.score))
        return ks, sc, bk

    def resident(self):
        """dict bucket -> set of resident keys."""
        ks, sc, bk = self._arrays()
        if ks.size == 0:
            return {}
        order = np.lexsort((ks, sc, bk))  # by bucket, then score, then key (ascending)
        ks, bk = ks[order], bk[order]
        _, start, counts = np.unique(bk, return_index=True, return_counts=True)
        keep = np.zeros(ks.size, dtype=bool)
        for s, c in zip(start, counts):
            lo = s + max(0, c - SLOTS)
            keep[lo:s + c] = True
        out = {}
        for k, b in zip(ks[keep].tolist(), bk[keep].tolist()):
            out.setdefault(b, set()).add(k)
        return out

    def resident_keys(self):
        s = set()
        for v in self.resident().values():
            s |= v
        return s

    def size(self):
        return sum(len(v) for v in self.resident().values())


def group_by_bucket(keys, pos) -> dict:
    """Exported (key, position) pairs -> dict bucket -> set of keys."""
    out = {}
    for k, p in zip(as_u64(keys).tolist(), as_u64(pos).tolist()):
        out.setdefault(p // SLOTS, set()).add(k)
    return out
