"""Seeded random small configurations: the HIP table against the CPU oracle,
exact, through the C ABI.

Each case draws a bucket count (powers of two and not, down to one bucket), a
row width (scalar and 16-byte copy paths, rows above 128 floats), a score
scheme (all equal, one score per call, jittered) and a sequence of calls of
every kind with batch sizes from one key to three times the capacity. Scores
never decrease for a key, so every call's result is the same in any order of
its keys and single-bucket mode is compared exactly after every call:
per-bucket contents, rows and scores, find outputs (misses untouched),
insert_and_evict's hand-back as a set, find_or_insert's flags and rows, and
each call's outcome counts (set differences of the oracle's states before and
after it; zero for the reader and updater calls).
In serial insert mode (single and dual bucket) scores are arbitrary and
every key's slot position is compared as well. Dual-bucket parallel mode is
held to its invariants after every call.
"""

import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from conftest import gpu_available
from helpers import SLOTS
from test_gpu_next_ops import evict_sets, oracle_evict_sets
from test_gpu_parity import assert_same_contents, check_find, dev, hkv, np_u64, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CALLS = ["insert_or_assign", "assign", "insert_and_evict", "find_or_insert", "find"]


def scheme_scores(scheme, rng, step, n):
    if scheme == "constant":
        return np.full(n, 7, np.uint64)
    if scheme == "step":
        return np.full(n, step, np.uint64)
    return (step * 1000 + rng.integers(0, 1000, size=n)).astype(np.uint64)


@pytest.mark.parametrize("case", range(24))
def test_random_small_configuration_exact(case):
    H = hkv()
    rng = np.random.default_rng(5000 + case)
    B = int(rng.choice([1, 2, 3, 5, 8, 13]))
    D = int(rng.choice([1, 2, 4, 7, 16, 64, 132]))
    scheme = str(rng.choice(["constant", "step", "jitter"]))
    C = B * SLOTS
    tab = H.HashTable(C, D)
    tab.count_outcomes()
    was = tab.outcomes()
    o = oracle.OracleTable(C, D)
    pool = gen.unique_keys(case, 7, 0, int(C * rng.uniform(0.5, 4.0)) + 1).numpy().view(np.uint64)
    absent = gen.unique_keys(case, 8, 0, 64).numpy().view(np.uint64)
    calls = int(rng.integers(4, 10))
    for step in range(1, calls + 1):
        # the first call always inserts, so that later calls meet residents
        call = "insert_or_assign" if step == 1 else str(rng.choice(CALLS))
        n = int(rng.integers(1, min(pool.size, 3 * C) + 1))
        k = rng.choice(pool, size=n, replace=False)
        kt = to_dev(k)
        sc = scheme_scores(scheme, rng, step, n)
        sct = to_dev(sc)
        v = gen.values(kt, 100 * case + step, D)
        print(f"case {case}: B={B} D={D} scheme={scheme} step={step} call={call} n={n}", flush=True)
        before = set(o.export()["keys"].tolist())
        if call == "insert_or_assign":
            tab.insert_or_assign(kt, v, sct)
            o.insert_or_assign(k, sc, values=v.cpu().numpy())
        elif call == "assign":
            # rows only, scores only, or both
            what = int(rng.integers(0, 3))
            tab.assign(kt, v if what != 1 else None, sct if what != 0 else None)
            o.assign(k, values=v.cpu().numpy() if what != 1 else None, scores=sc if what != 0 else None)
        elif call == "insert_and_evict":
            got = evict_sets(*tab.insert_and_evict(kt, v, sct))
            want = oracle_evict_sets(o.insert_and_evict(k, sc, values=v.cpu().numpy()))
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
            assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        elif call == "find_or_insert":
            v0 = v.cpu().numpy()
            rows, found = tab.find_or_insert(kt, v, sct)
            orows, ofound = o.find_or_insert(k, sc, values=v0)
            torch.cuda.synchronize()
            assert np.array_equal(found.cpu().numpy(), ofound)
            assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        else:
            q = np.random.default_rng(case * 100 + step).permutation(np.concatenate([k[: max(1, n // 2)], absent]))
            check_find(tab, o, to_dev(q))
        assert_same_contents(tab, o)
        after = set(o.export()["keys"].tolist())
        now = tab.outcomes()
        want = dict(updated=0, inserted=0, evicted=0, rejected=0)
        if call in ("insert_or_assign", "insert_and_evict", "find_or_insert"):
            b = set(k.tolist())
            want = dict(updated=len(b & before), inserted=len(after - before), evicted=len(before - after),
                        rejected=len(b - before - after))
        assert {x: now[x] - was[x] for x in now} == want
        was = now


def assert_same_positions(tab, o):
    gk, _, gs, gp = tab.export_batch(with_values=False)
    e = o.export()
    order = np.argsort(np_u64(gp))
    assert np.array_equal(np_u64(gp)[order], e["pos"])
    assert np.array_equal(np_u64(gk)[order], e["keys"])
    assert np.array_equal(np_u64(gs)[order], e["scores"])


@pytest.mark.parametrize("dual", [False, True])
@pytest.mark.parametrize("case", range(8))
def test_random_serial_mode_positions_exact(case, dual):
    """Serial insert mode applies keys in input order, as the oracle does, so
    scores may be anything: drawn from a small range, with ties everywhere and
    updates that lower a key's score. Every key must sit in the oracle's slot
    (Algorithms 2 and 3) after every call; insert_and_evict hands back the
    oracle's departures in the oracle's order."""
    H = hkv()
    rng = np.random.default_rng(7000 + case + 100 * dual)
    B = int(rng.choice([1, 2, 3, 5, 8]))
    D = int(rng.choice([1, 4, 7, 64]))
    C = B * SLOTS
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=dual)
    pool = gen.unique_keys(case + 50 * dual, 9, 0, int(C * rng.uniform(0.5, 3.0)) + 1).numpy().view(np.uint64)
    absent = gen.unique_keys(case, 10, 0, 64).numpy().view(np.uint64)
    for step in range(1, int(rng.integers(4, 9)) + 1):
        call = "insert_or_assign" if step == 1 else str(rng.choice(CALLS))
        n = int(rng.integers(1, min(pool.size, 2 * C) + 1))
        k = rng.choice(pool, size=n, replace=False)
        kt = to_dev(k)
        sc = rng.integers(0, 50, size=n).astype(np.uint64)
        sct = to_dev(sc)
        v = gen.values(kt, 100 * case + step, D)
        print(f"serial case {case} dual={dual}: B={B} D={D} step={step} call={call} n={n}", flush=True)
        if call == "insert_or_assign":
            tab.insert_or_assign(kt, v, sct)
            o.insert_or_assign(k, sc, values=v.cpu().numpy())
        elif call == "assign":
            tab.assign(kt, v, sct)
            o.assign(k, values=v.cpu().numpy(), scores=sc)
        elif call == "insert_and_evict":
            ek, ev, es, cnt = tab.insert_and_evict(kt, v, sct)
            want = o.insert_and_evict(k, sc, values=v.cpu().numpy())
            torch.cuda.synchronize()
            m = int(cnt.item())
            assert np.array_equal(np_u64(ek[:m]), want["keys"])
            assert np.array_equal(np_u64(es[:m]), want["scores"])
            assert np.array_equal(ev[:m].cpu().numpy().view(np.uint32), want["values"].view(np.uint32))
        elif call == "find_or_insert":
            v0 = v.cpu().numpy()
            rows, found = tab.find_or_insert(kt, v, sct)
            orows, ofound = o.find_or_insert(k, sc, values=v0)
            torch.cuda.synchronize()
            assert np.array_equal(found.cpu().numpy(), ofound)
            assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        else:
            q = np.random.default_rng(case * 100 + step).permutation(np.concatenate([k[: max(1, n // 2)], absent]))
            check_find(tab, o, to_dev(q))
        assert_same_positions(tab, o)
    assert_same_contents(tab, o)


@pytest.mark.parametrize("case", range(12))
def test_random_dual_parallel_invariants(case):
    """Dual-bucket parallel mode picks among equally valid placements, so it is
    held to invariants after every call of a random sequence: no key twice, at
    most 128 per bucket, every entry in one of its two candidate buckets, each
    resident key's score and row its last written ones, find hitting exactly
    the resident keys, and insert_and_evict's hand-back and the table together
    holding exactly what was resident or offered; each call's outcome counts
    equal the set differences of the table's states before and after it."""
    H = hkv()
    rng = np.random.default_rng(9000 + case)
    B = int(rng.choice([2, 3, 5, 8, 13]))
    D = int(rng.choice([1, 4, 7, 64]))
    C = B * SLOTS
    tab = H.HashTable(C, D, dual_bucket=True)
    tab.count_outcomes()
    was = tab.outcomes()
    route = oracle.OracleTable(SLOTS * B, 1, dual=True)  # routing only
    pool = gen.unique_keys(case + 200, 11, 0, int(C * rng.uniform(0.5, 3.0)) + 1).numpy().view(np.uint64)
    absent = gen.unique_keys(case + 200, 12, 0, 64).numpy().view(np.uint64)
    last_score, last_row = {}, {}
    resident = set()

    def rows_of(keys_u64):
        ver = np.array([last_row[int(x)] for x in keys_u64.tolist()], dtype=np.int64)
        return gen.values(to_dev(keys_u64), torch.from_numpy(ver).to(dev()), D)

    for step in range(1, int(rng.integers(4, 10)) + 1):
        call = "insert_or_assign" if step == 1 else str(rng.choice(CALLS))
        n = int(rng.integers(1, min(pool.size, 3 * C) + 1))
        k = rng.choice(pool, size=n, replace=False)
        kt = to_dev(k)
        sc = (step * 1000 + rng.integers(0, 1000, size=n)).astype(np.uint64)
        sct = to_dev(sc)
        ver = torch.full((n,), 1000 * case + step, dtype=torch.int64, device=dev())
        v = gen.values(kt, ver, D)
        print(f"dual case {case}: B={B} D={D} step={step} call={call} n={n}", flush=True)
        before = set(resident)
        if call == "find":
            q = np.random.default_rng(case * 100 + step).permutation(np.concatenate([k[: max(1, n // 2)], absent]))
            vals, found, scs = tab.find(to_dev(q), with_scores=True)
            f = found.cpu().numpy().astype(bool)
            assert np.array_equal(f, np.array([int(x) in resident for x in q.tolist()]))
            hit = q[f]
            assert np.array_equal(np_u64(scs)[f], np.array([last_score[int(x)] for x in hit.tolist()], np.uint64))
            if hit.size:
                assert torch.equal(vals[torch.from_numpy(f).to(dev())], rows_of(hit))
            continue
        if call == "assign":
            tab.assign(kt, v, sct)
            for x, s in zip(k.tolist(), sc.tolist()):
                if x in resident:
                    last_score[x], last_row[x] = s, 1000 * case + step
        elif call == "find_or_insert":
            rows, found = tab.find_or_insert(kt, v, sct)
            f = found.cpu().numpy().astype(bool)
            assert np.array_equal(f, np.array([int(x) in before for x in k.tolist()]))
            if f.any():
                assert torch.equal(rows[torch.from_numpy(f).to(dev())], rows_of(k[f]))
            for x, s, hit_ in zip(k.tolist(), sc.tolist(), f.tolist()):
                last_score[x] = s
                if not hit_:
                    last_row[x] = 1000 * case + step
        else:
            for x, s in zip(k.tolist(), sc.tolist()):
                last_score[x], last_row[x] = s, 1000 * case + step
            if call == "insert_or_assign":
                tab.insert_or_assign(kt, v, sct)
            else:
                ek, ev, es, cnt = tab.insert_and_evict(kt, v, sct)
                torch.cuda.synchronize()
                m = int(cnt.item())
                out = np_u64(ek[:m])
                assert np.unique(out).size == m
                assert np.array_equal(np_u64(es[:m]), np.array([last_score[int(x)] for x in out.tolist()], np.uint64))
                if m:
                    assert torch.equal(ev[:m], rows_of(out))
        gk, gv, gs, gp = tab.export_batch()
        k_, s_, p_ = np_u64(gk), np_u64(gs), np_u64(gp)
        resident = set(k_.tolist())
        assert np.unique(k_).size == k_.size and tab.size() == k_.size <= C
        assert np.bincount((p_ // SLOTS).astype(np.int64), minlength=B).max() <= SLOTS
        b1, b2, _ = route.route(k_)
        assert np.all((p_ // SLOTS == b1) | (p_ // SLOTS == b2))
        assert np.array_equal(s_, np.array([last_score[int(x)] for x in k_.tolist()], np.uint64))
        if k_.size:
            assert torch.equal(gv, rows_of(k_))
        offered = set(k.tolist())
        if call == "insert_and_evict":
            assert not (set(out.tolist()) & resident)
            assert set(out.tolist()) | resident == before | offered
        elif call in ("insert_or_assign", "find_or_insert"):
            assert resident <= before | offered
        else:
            assert resident == before
        now = tab.outcomes()
        want = dict(updated=0, inserted=0, evicted=0, rejected=0)
        if call != "assign":
            want = dict(updated=len(offered & before), inserted=len(resident - before),
                        evicted=len(before - resident), rejected=len(offered - before - resident))
        assert {x: now[x] - was[x] for x in now} == want
        was = now


@pytest.mark.parametrize("lanes,keys_per_group", [("4", "1"), ("16", "4"), ("4", "4"), ("16", "1")])
@pytest.mark.parametrize("dual", [False, True])
def test_tuning_overrides_keep_results_exact(lanes, keys_per_group, dual, monkeypatch):
    """HKV_GROUP_LANES and HKV_KEYS_PER_GROUP change only launch shapes: the
    probing kernels at 4 and 16 lanes per key and the key-side probes at 1
    and 4 keys per group give the oracle's results (serial mode in dual, for
    exact positions)."""
    monkeypatch.setenv("HKV_GROUP_LANES", lanes)
    monkeypatch.setenv("HKV_KEYS_PER_GROUP", keys_per_group)
    H = hkv()
    B, D = 5, 40  # 160-byte rows: 8 lanes by default, so both overrides change the shape
    C = B * SLOTS
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=dual)
    o = oracle.OracleTable(C, D, dual=dual)
    pool = gen.unique_keys(31, 13, 0, 3 * C).numpy().view(np.uint64)
    absent = gen.unique_keys(31, 14, 0, 200).numpy().view(np.uint64)
    rng = np.random.default_rng(int(lanes) * 10 + int(keys_per_group) + dual)
    for step in range(1, 5):
        k = rng.choice(pool, size=C, replace=False)
        kt = to_dev(k)
        sc = np.full(C, step, np.uint64)
        v = gen.values(kt, step, D)
        tab.insert_or_assign(kt, v, to_dev(sc))
        o.insert_or_assign(k, sc, values=v.cpu().numpy())
        assert_same_contents(tab, o)
        if dual:
            assert_same_positions(tab, o)
        q = rng.permutation(np.concatenate([rng.choice(pool, 333, replace=False), absent]))
        qt = to_dev(q)
        check_find(tab, o, qt)
        ptrs = torch.zeros(q.size, dtype=torch.int64, device=dev())
        found = torch.empty(q.size, dtype=torch.uint8, device=dev())
        tab.find_ptr(qt, ptrs_out=ptrs, found_out=found)
        contains = tab.contains(qt)
        torch.cuda.synchronize()
        ofound, _ = o.find_pos(q)
        assert np.array_equal(found.cpu().numpy(), ofound)
        assert np.array_equal(contains.cpu().numpy(), ofound)
        assert np.all((ptrs.cpu().numpy() != 0) == ofound.astype(bool))
