"""The contents of a single-bucket table at any size, from its plain definition.

With distinct keys per write batch and scores that never decrease per key,
the bucket-local admission and eviction of §3.3 (Algorithm 2 of the
HierarchicalKV paper) reach a state that has a closed form: bucket b holds
exactly the min(128, m_b) keys ranked highest by (latest score, key) among
the m_b distinct keys ever routed to b by insert_or_assign. An updater that
raises the score of a resident key leaves that set as it is and only moves
the key up.

This module writes that definition out with library sorts over every offered
key (on whatever device the tensors live on), so that tables of 2^26-2^28
slots can be compared with it bucket by bucket, all buckets. Bucket routing
comes from the oracle's route function; nothing here uses the HIP library.
64-bit keys and scores are int64 tensors holding the unsigned bit patterns.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

SLOTS = 128
_SIGN = -(1 << 63)


def lex_order(major: torch.Tensor, key: torch.Tensor) -> torch.Tensor:
    """Permutation that sorts by (major, key), major a non-negative int64 and
    key compared as an unsigned 64-bit word."""
    o = torch.argsort(key ^ _SIGN, stable=True)
    return o[torch.argsort(major[o], stable=True)]


def buckets_of(keys: torch.Tensor, capacity: int) -> torch.Tensor:
    """First-choice bucket of every key (the oracle's routing), on keys' device."""
    b1, _, _ = oracle.route_buckets(keys.cpu().numpy().view(np.uint64), capacity // SLOTS, False)
    return torch.from_numpy(b1.view(np.int64)).to(keys.device)


def expected_contents(keys: torch.Tensor, scores: torch.Tensor, capacity: int, buckets: torch.Tensor | None = None):
    """(buckets, keys) of every entry the table must hold, sorted by (bucket,
    key). keys: every distinct key ever offered to insert_or_assign; scores:
    its latest score (non-negative, below 2^31); buckets: the keys' buckets
    when already known (buckets_of)."""
    assert keys.numel() == scores.numel()
    assert int(scores.min()) >= 0 and int(scores.max()) < (1 << 31)
    nb = capacity // SLOTS
    b = buckets_of(keys, capacity) if buckets is None else buckets
    o = lex_order(b * (1 << 31) + scores, keys)  # by (bucket, score, key)
    bs, ks = b[o], keys[o]
    ends = torch.cumsum(torch.bincount(bs, minlength=nb), 0)
    j = torch.arange(bs.numel(), device=bs.device)
    keep = j >= ends[bs] - SLOTS  # the last (highest) min(128, m_b) of each bucket's run
    eb, ek = bs[keep], ks[keep]
    o2 = lex_order(eb, ek)
    return eb[o2], ek[o2]


def assert_table_matches(export_keys: torch.Tensor, export_pos: torch.Tensor, keys: torch.Tensor,
                         scores: torch.Tensor, capacity: int, buckets: torch.Tensor | None = None) -> torch.Tensor:
    """Every bucket of an exported table holds exactly the closed form's set.
    Returns the closed form's resident keys sorted as signed int64 (for
    torch.searchsorted membership tests)."""
    eb, ek = expected_contents(keys, scores, capacity, buckets)
    gb = torch.div(export_pos, SLOTS, rounding_mode="floor")
    o = lex_order(gb, export_keys)
    gb, gk = gb[o], export_keys[o]
    assert gk.numel() == ek.numel(), f"table holds {gk.numel()} entries, closed form {ek.numel()}"
    if not (torch.equal(gb, eb) and torch.equal(gk, ek)):
        bad = torch.nonzero((gb != eb) | (gk != ek)).flatten()
        first = int(bad[0])
        raise AssertionError(f"{bad.numel()} entries differ from the closed form; first at sorted index {first}: "
                             f"table (bucket {int(gb[first])}, key {int(gk[first]) & ((1 << 64) - 1):#x}), "
                             f"closed form (bucket {int(eb[first])}, key {int(ek[first]) & ((1 << 64) - 1):#x})")
    return torch.sort(ek).values


def resident_keys(keys: torch.Tensor, scores: torch.Tensor, capacity: int,
                  buckets: torch.Tensor | None = None) -> torch.Tensor:
    """The resident keys by the closed form, sorted as signed int64 (for
    torch.searchsorted membership tests)."""
    _, ek = expected_contents(keys, scores, capacity, buckets)
    return torch.sort(ek).values


class FillCount:
    """Size of a single-bucket table by the closed form while it is filled
    with keys never offered before: sum over buckets of min(128, m_b)."""

    def __init__(self, capacity: int, device):
        self.capacity = capacity
        self.m = torch.zeros(capacity // SLOTS, dtype=torch.int64, device=device)

    def add(self, fresh_keys: torch.Tensor) -> int:
        self.m += torch.bincount(buckets_of(fresh_keys, self.capacity), minlength=self.m.numel())
        return self.size()

    def size(self) -> int:
        return int(torch.clamp(self.m, max=SLOTS).sum())
