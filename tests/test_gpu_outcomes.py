"""Outcome counters of the inserter calls (hkv_set_outcome_counters).

For a batch B of distinct keys the four counts are properties of the call's
start state S0 and end state S1 alone:
  updated = |B ∩ S0|, inserted = |S1 − S0|, evicted = |S0 − S1|,
  rejected = |B − S0 − S1|.
In single-bucket mode the end state is the oracle's (checked here too), so
the expected counts come from the oracle's exports before and after each
call. In dual-bucket parallel mode, which is not the sequential oracle's
order, they come from the GPU table's own exports before and after.
"""

import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SLOTS = 128


def dev():
    return torch.device("cuda", 0)


def hkv():
    import hash_table_cache_amd

    return hash_table_cache_amd


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).to(dev())


def u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def gpu_keys(tab):
    k, _, _, _ = tab.export_batch(with_values=False)
    return set(u64(k).tolist())


def expected(batch, before, after):
    b = set(batch.tolist())
    return {"updated": len(b & before), "inserted": len(after - before), "evicted": len(before - after),
            "rejected": len(b - before - after)}


def delta(now, was):
    return {k: now[k] - was[k] for k in now}


def call(kind, tab, o, k, sc, step, D):
    """One inserter call of `kind` on the GPU table and (when given) the oracle."""
    kt, st = to_dev(k), to_dev(sc)
    v = gen.values(kt, step, D)
    if kind == "insert_or_assign":
        tab.insert_or_assign(kt, v, st)
        if o is not None:
            o.insert_or_assign(k, sc, values=v.cpu().numpy())
    elif kind == "insert_and_evict":
        tab.insert_and_evict(kt, v, st)
        if o is not None:
            o.insert_and_evict(k, sc, values=v.cpu().numpy())
    else:
        tab.find_or_insert(kt, v.clone(), st)
        if o is not None:
            o.find_or_insert(k, sc, values=v.cpu().numpy())


KINDS = ("insert_or_assign", "insert_and_evict", "find_or_insert")


@pytest.mark.parametrize("unique_keys", [False, True])
def test_counts_single_bucket_match_the_oracle(unique_keys):
    """16 buckets, dim 8; every batch sends its keys to 4 of them (long
    chains, evictions, rejections, in-call displacement), mixing resident
    keys with new ones; scores rise with the step and jitter within it (ties
    broken by key). Nine calls, three of each inserter."""
    H = hkv()
    C, D = 16 * SLOTS, 8
    tab = H.HashTable(C, D, unique_keys=unique_keys)
    o = oracle.OracleTable(C, D)
    tab.count_outcomes()
    rng = np.random.default_rng(90)
    cand = rng.integers(1, 1 << 62, size=300000, dtype=np.int64).view(np.uint64)
    hot = cand[np.isin(o.route(cand)[0], [1, 6, 9, 14])]
    cursor = 0
    was = tab.outcomes()
    for step in range(1, 10):
        before = set(o.export()["keys"].tolist())
        res = np.array(sorted(before), dtype=np.uint64)
        old = rng.choice(res, size=min(150, res.size), replace=False) if res.size else np.zeros(0, np.uint64)
        fresh = hot[cursor: cursor + 260]
        cursor += 260
        k = rng.permutation(np.concatenate([old, fresh]))
        sc = (step * 8 + rng.integers(0, 8, size=k.size)).astype(np.uint64)
        call(KINDS[(step - 1) % 3], tab, o, k, sc, step, D)
        after = set(o.export()["keys"].tolist())
        assert gpu_keys(tab) == after
        now = tab.outcomes()
        assert delta(now, was) == expected(k, before, after), f"step {step} ({KINDS[(step - 1) % 3]})"
        was = now
    assert tab.size() == len(after)
    tab.close()


def test_counts_dual_bucket_match_the_table_states():
    """Dual-bucket parallel mode: counts equal the set differences of the
    table's own states before and after each call (Zipf-drawn batches, LFU
    scores, a table driven past full)."""
    H = hkv()
    C, D = 32 * SLOTS, 4
    tab = H.HashTable(C, D, dual_bucket=True)
    tab.count_outcomes()
    zipf = gen.Zipf(1.05, 1 << 16)
    freq = torch.zeros((1 << 16) + 1, dtype=torch.int64, device=dev())
    was = tab.outcomes()
    for step in range(12):
        r = zipf.draw(0x5EED, 3, step * 3000, 3000, device=dev())
        uniq, cnt = torch.unique(r, return_counts=True)
        freq.index_add_(0, uniq, cnt)
        k, sc = u64(uniq), u64(freq[uniq])
        before = gpu_keys(tab)
        call(KINDS[step % 3], tab, None, k, sc, step, D)
        after = gpu_keys(tab)
        now = tab.outcomes()
        assert delta(now, was) == expected(k, before, after), f"step {step} ({KINDS[step % 3]})"
        was = now
    tab.close()


@pytest.mark.parametrize("dual", [False, True])
def test_counts_with_repeated_keys(dual):
    """A third of each insert_or_assign batch repeats other keys of the batch
    (claims on): a resident key is counted updated once; inserted and evicted
    are the set differences; size after = size before + inserted - evicted."""
    H = hkv()
    C, D = 16 * SLOTS, 64
    tab = H.HashTable(C, D, dual_bucket=dual)
    tab.count_outcomes()
    rng = np.random.default_rng(91)
    pool = rng.integers(1, 1 << 62, size=3 * C, dtype=np.int64).view(np.uint64)
    was = tab.outcomes()
    for step in range(1, 7):
        base = rng.choice(pool, size=C // 2, replace=False)
        k = rng.permutation(np.concatenate([base, rng.choice(base, size=C // 4)]))
        sc = np.full(k.size, step, dtype=np.uint64)
        before = gpu_keys(tab)
        call("insert_or_assign", tab, None, k, sc, step, D)
        after = gpu_keys(tab)
        now = tab.outcomes()
        d = delta(now, was)
        want = expected(np.unique(k), before, after)
        assert (d["updated"], d["inserted"], d["evicted"]) == (want["updated"], want["inserted"], want["evicted"])
        assert len(after) == len(before) + d["inserted"] - d["evicted"]
        was = now
    tab.close()


@pytest.mark.parametrize("kind", KINDS)
def test_reserved_keys_count_in_no_outcome(kind):
    """The reserved keys (2^64 - 1, 2^64 - 2) are skipped by every inserter:
    a batch that carries them among resident and new keys counts only the
    others."""
    H = hkv()
    C, D = 8 * SLOTS, 4
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    tab.count_outcomes()
    old = np.arange(1, 201, dtype=np.uint64)
    call("insert_or_assign", tab, o, old, np.ones(200, np.uint64), 1, D)
    was = tab.outcomes()
    rsv = np.array([2**64 - 1, 2**64 - 2, 2**64 - 1], dtype=np.uint64)
    k = np.random.default_rng(92).permutation(np.concatenate([rsv, old[:50], np.arange(1000, 1040, dtype=np.uint64)]))
    before = set(o.export()["keys"].tolist())
    call(kind, tab, o, k, np.full(k.size, 2, np.uint64), 2, D)
    after = set(o.export()["keys"].tolist())
    assert gpu_keys(tab) == after
    d = delta(tab.outcomes(), was)
    assert d == expected(k[k < 2**64 - 2], before, after) == {"updated": 50, "inserted": 40, "evicted": 0,
                                                                "rejected": 0}
    tab.close()


def test_counting_off_serial_tables_and_bad_arguments():
    H = hkv()
    C, D = 4 * SLOTS, 4
    tab = H.HashTable(C, D)
    tab.count_outcomes()
    k = to_dev(np.arange(1, 301, dtype=np.uint64))
    sc = torch.ones(300, dtype=torch.int64, device=dev())
    tab.insert_or_assign(k, gen.values(k, 1, D), sc)
    assert tab.outcomes() == {"updated": 0, "inserted": 300, "evicted": 0, "rejected": 0}
    tab.insert_or_assign(k[:0], gen.values(k[:0], 1, D), sc[:0])  # an empty batch counts nothing
    assert tab.outcomes()["inserted"] == 300
    tab.count_outcomes(False)
    tab.insert_or_assign(k, gen.values(k, 2, D), sc + 1)
    with pytest.raises(RuntimeError):
        tab.outcomes()
    with pytest.raises(H.HkvError):  # pinned host memory is not device memory of the GPU
        H.hkv_set_outcome_counters(tab._h, torch.zeros(4, dtype=torch.int64).pin_memory())
    with pytest.raises(ValueError):
        H.hkv_set_outcome_counters(tab._h, torch.zeros(3, dtype=torch.int64, device=dev()))
    tab.close()
    serial = H.HashTable(C, D, serial_insert=True)
    with pytest.raises(H.HkvError, match="serial"):
        serial.count_outcomes()
    serial.close()
