"""Pins of the test-side closed form (tests/closed_form.py) that the
full-size GPU tests compare whole tables with: on small tables it must give
exactly the oracle's per-bucket sets (the oracle applies Algorithm 2 key by
key and is pinned on its own), agree with a per-bucket brute force written
with Python sets, and notice a planted mistake. CPU only."""

import numpy as np
import pytest
import torch

import closed_form as cf
import hkv_inputs as gen
import oracle

SLOTS = 128


def u64(t):
    return t.numpy().view(np.uint64)


def workload(seed, capacity, batches, batch, dim=4):
    """Distinct uniform keys per batch, score = batch index, a third of each
    batch re-offering earlier keys (their score rises)."""
    o = oracle.OracleTable(capacity, dim)
    latest = {}
    rng = np.random.default_rng(seed)
    cursor = 0
    for step in range(1, batches + 1):
        fresh = gen.unique_keys(seed, 1, cursor, batch)
        cursor += batch
        old = list(latest)
        again = (torch.tensor(rng.choice(np.array(old, dtype=np.uint64), size=min(len(old), batch // 3),
                                         replace=False).view(np.int64)) if old else torch.empty(0, dtype=torch.int64))
        k = torch.cat([fresh, again])
        sc = torch.full((k.numel(),), step, dtype=torch.int64)
        o.insert_or_assign(u64(k), u64(sc), values=gen.values(k, step, dim).numpy())
        for key in u64(k).tolist():
            latest[key] = step
    keys = torch.tensor(np.array(list(latest), dtype=np.uint64).view(np.int64))
    scores = torch.tensor(list(latest.values()), dtype=torch.int64)
    return o, keys, scores


@pytest.mark.parametrize("capacity,batches,batch", [(8 * SLOTS, 6, 500), (64 * SLOTS, 5, 4000), (SLOTS, 4, 300)])
def test_closed_form_equals_the_oracle(capacity, batches, batch):
    o, keys, scores = workload(capacity + batches, capacity, batches, batch)
    e = o.export()
    ek = torch.from_numpy(e["keys"].view(np.int64).copy())
    ep = torch.from_numpy(e["pos"].view(np.int64).copy())
    resident = cf.assert_table_matches(ek, ep, keys, scores, capacity)
    assert torch.equal(resident, torch.sort(ek).values)


def test_closed_form_equals_brute_force():
    capacity = 4 * SLOTS
    rng = np.random.default_rng(3)
    keys = torch.tensor(rng.integers(-(1 << 63), (1 << 63) - 1, size=3000, dtype=np.int64))
    keys = torch.unique(keys)
    scores = torch.tensor(rng.integers(0, 5, size=keys.numel()), dtype=torch.int64)  # many ties
    eb, ek = cf.expected_contents(keys, scores, capacity)
    b1, _, _ = oracle.route_buckets(u64(keys), capacity // SLOTS)
    want = set()
    for b in range(capacity // SLOTS):
        members = [(int(s), int(k) & ((1 << 64) - 1)) for k, s, bb in zip(keys.tolist(), scores.tolist(), b1.tolist())
                   if bb == b]
        members.sort()
        want |= {(b, k) for _, k in members[-SLOTS:]}
    got = {(int(b), int(k) & ((1 << 64) - 1)) for b, k in zip(eb.tolist(), ek.tolist())}
    assert got == want
    assert len(got) == ek.numel()


def test_closed_form_notices_a_swapped_entry():
    capacity = 8 * SLOTS
    o, keys, scores = workload(9, capacity, 5, 500)
    e = o.export()
    ek = torch.from_numpy(e["keys"].view(np.int64).copy())
    ep = torch.from_numpy(e["pos"].view(np.int64).copy())
    # one resident entry replaced by a departed key of the same bucket
    b1, _, _ = oracle.route_buckets(u64(keys), capacity // SLOTS)
    res = set(u64(ek).tolist())
    gone = [(k, b) for k, b in zip(u64(keys).tolist(), b1.tolist()) if k not in res]
    assert gone, "the workload evicts or rejects some keys"
    k_out, b_out = gone[0]
    j = int(torch.nonzero(torch.div(ep, SLOTS, rounding_mode="floor") == b_out)[0])
    bad = ek.clone()
    bad[j] = int(np.uint64(k_out).view(np.int64))
    with pytest.raises(AssertionError):
        cf.assert_table_matches(bad, ep, keys, scores, capacity)
    # and a lowered score moves the boundary of a full bucket
    low = scores.clone()
    low[torch.nonzero(keys == ek[0])[0]] = 0
    with pytest.raises(AssertionError):
        cf.assert_table_matches(ek, ep, keys, low, capacity)
