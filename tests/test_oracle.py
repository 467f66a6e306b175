"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what it checks and where the fact comes from ("paper" is
"HierarchicalKV: A GPU Hash Table with Cache Semantics for Continuous Online
Embedding Storage", arXiv 2603.17168):

* fmix64: SMHasher's published MurmurHash3_x64_128 verification value.
* routing: the digest reading (bits 32..39), bucket = hash mod B, uniformity.
* single-bucket contents: the closed form (top-128 by (score, key) per bucket)
  computed by an independent model, on tiny tables, adversarial one-bucket
  streams, and the tiny single-bucket workload (512 buckets, dim 16).
* find outputs: hit iff resident, last-written value and score; misses leave
  outputs untouched (§3.2, Algorithm 1).
* admission (§5.4, Table 9): a low-score burst into a loaded table displaces
  nobody; a high-score burst is admitted in full.
* find* / contains (§4.1, §5.3): positions agree with export and routing;
  insert_and_evict hands back exactly (resident before ∪ offered) − resident
  after, with last-written rows and scores; find_or_insert returns stored rows
  for hits and inserts misses as insert_or_assign does (closed form).
* Proposition 3.1: about 0.5 false-positive key compares per miss.
* Proposition 3.3: evicting from the bucket with the lower minimum halves the
  expected evicted score (1/(2n+1) vs 1/(n+1), n = 128).
* Algorithm 3 step by step, restated as the minimum over the union of the two
  candidate buckets; first-eviction load factor of dual vs single (§3.4).
"""

import math
import pathlib

import hypothesis
import hypothesis.strategies as st
import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from helpers import SLOTS, TopKModel, as_u64, group_by_bucket

GOLDEN = pathlib.Path(__file__).parent / "golden"


def u64(x):
    return np.asarray(x, dtype=np.uint64)


def rand_keys(rng, n, lo=1, hi=1 << 62):
    return u64(rng.integers(lo, hi, size=n, dtype=np.int64))


# --------------------------------------------------------------- routing ----

def test_fmix64_pinned_by_smhasher_verification_value():
    line = [l for l in (GOLDEN / "smhasher_murmur3_x64_128.txt").read_text().splitlines()
            if l.startswith("verification")][0]
    expected = int(line.split()[1], 16)
    key = bytearray(256)
    hashes = bytearray()
    for i in range(256):
        key[i] = i
        h1, h2 = oracle.murmur3_x64_128(bytes(key[:i]), 256 - i)
        hashes += h1.to_bytes(8, "little") + h2.to_bytes(8, "little")
    f1, _ = oracle.murmur3_x64_128(bytes(hashes), 0)
    assert f1 & 0xFFFFFFFF == expected


def test_fmix64_fixed_point_and_avalanche():
    assert oracle.fmix64(0) == 0
    rng = np.random.default_rng(1)
    flips = []
    for _ in range(400):
        x = int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2))
        b = int(rng.integers(0, 64))
        flips.append(bin(oracle.fmix64(x) ^ oracle.fmix64(x ^ (1 << b))).count("1"))
    assert 30 < np.mean(flips) < 34


def test_route_reading_bits_and_modulo():
    t = oracle.OracleTable(capacity=128 * 6, dim=1, dual=True)  # B = 6: not a power of two
    rng = np.random.default_rng(2)
    keys = rand_keys(rng, 2000)
    b1, b2, d = t.route(keys)
    for k, x1, x2, dd in zip(keys.tolist(), b1.tolist(), b2.tolist(), d.tolist()):
        h = oracle.fmix64(k)
        assert x1 == h % 6
        assert dd == (h >> 32) & 0xFF  # digest = bits 32..39 (reading of §3.2)
        assert x2 == oracle.fmix64(k ^ 0x9E3779B97F4A7C15) % 6


def test_route_uniform_over_buckets():
    t = oracle.OracleTable(capacity=128 * 256, dim=1)
    keys = gen.unique_keys(7, 1, 0, 256 * 400).numpy().view(np.uint64)
    b1, _, d = t.route(keys)
    counts = np.bincount(b1.astype(np.int64), minlength=256)
    chi2 = ((counts - 400) ** 2 / 400).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)
    dc = np.bincount(d.astype(np.int64), minlength=256)
    chi2d = ((dc - 400) ** 2 / 400).sum()
    assert chi2d < 255 + 6 * math.sqrt(2 * 255)


# ------------------------------------------------- single-bucket contents --

def oracle_buckets(t):
    e = t.export()
    return group_by_bucket(e["keys"], e["pos"])


def check_against_model(t, model, dim):
    res = model.resident()
    got = oracle_buckets(t)
    assert got == res
    assert t.size() == model.size()
    e = t.export()
    for k, s, v in zip(e["keys"].tolist(), e["scores"].tolist(), e["values"]):
        assert model.score[k] == s
        np.testing.assert_array_equal(v, model.payload[k])


def random_workload(seed, B, dim, batches, batch, key_pool, tie_heavy):
    rng = np.random.default_rng(seed)
    t = oracle.OracleTable(capacity=B * SLOTS, dim=dim)
    model = TopKModel(lambda k: t.route(k)[0], dim)
    pool = rand_keys(rng, key_pool)
    step = 0
    for _ in range(batches):
        keys = rng.choice(pool, size=min(batch, key_pool), replace=False)
        step += 1
        if tie_heavy:
            scores = u64(np.full(keys.size, step))
        else:
            # non-decreasing per key over time: step * 1000 + jitter
            scores = u64(step * 1000 + rng.integers(0, 1000, size=keys.size))
        vals = rng.standard_normal((keys.size, dim)).astype(np.float32)
        out = t.insert_or_assign(keys, scores, values=vals)
        assert set(np.unique(out).tolist()) <= {oracle.UPDATED, oracle.INSERTED, oracle.EVICTED, oracle.REJECTED}
        model.insert_or_assign(keys, scores, vals)
        check_against_model(t, model, dim)
    return t, model


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("tie_heavy", [False, True])
def test_single_bucket_topk_tiny_tables(B, tie_heavy):
    random_workload(10 + B, B, 3, batches=12, batch=150 * B, key_pool=600 * B, tie_heavy=tie_heavy)


# Score schemes for the property test below. Each keeps every key's score
# non-decreasing over time, the condition under which the table's contents
# equal the top 128 by (score, key) of everything ever offered to a bucket:
# a key that was evicted or rejected sits below a bucket minimum that never
# falls again.
def _scores(scheme, rng, step, n):
    if scheme == "constant":        # every key the same score forever
        return u64(np.full(n, 7))
    if scheme == "step":            # one score per batch: ties inside it
        return u64(np.full(n, step))
    if scheme == "coarse":          # four levels per batch: many ties
        return u64(step * 4 + rng.integers(0, 4, size=n))
    return u64(step * 1000 + rng.integers(0, 1000, size=n))  # "jitter"


_ASSIGN_TOP = {"constant": lambda s: 7, "step": lambda s: s,
               "coarse": lambda s: s * 4 + 3, "jitter": lambda s: s * 1000 + 999}


@hypothesis.settings(max_examples=60, deadline=None, derandomize=True,
                     suppress_health_check=[hypothesis.HealthCheck.too_slow])
@hypothesis.given(
    seed=st.integers(0, 2**32 - 1),
    B=st.integers(1, 5),
    dim=st.sampled_from([1, 3]),
    batches=st.integers(1, 7),
    batch=st.integers(1, 420),
    pool_factor=st.sampled_from([1, 2, 4]),
    scheme=st.sampled_from(["constant", "step", "coarse", "jitter"]),
    with_assign=st.booleans(),
)
def test_single_bucket_topk_property(seed, B, dim, batches, batch, pool_factor, scheme, with_assign):
    """Random tiny tables (including bucket counts that are not powers of two,
    where routing is hash mod B), batch sizes from one key to more than three
    buckets' worth, and score streams from all-equal to jittered: after every
    insert_or_assign, and after every assign of raised scores, each bucket holds
    exactly the top 128 of its offered keys by (score, key) with the
    last-written row and score (the paper's cache semantics, §3.1 and §4.1),
    and find agrees with that set."""
    rng = np.random.default_rng(seed)
    t = oracle.OracleTable(capacity=B * SLOTS, dim=dim)
    model = TopKModel(lambda k: t.route(k)[0], dim)
    pool = np.unique(rand_keys(rng, max(1, batch * pool_factor)))
    for step in range(1, batches + 1):
        keys = rng.choice(pool, size=min(batch, pool.size), replace=False)
        sc = _scores(scheme, rng, step, keys.size)
        vals = rng.standard_normal((keys.size, dim)).astype(np.float32)
        t.insert_or_assign(keys, sc, values=vals)
        model.insert_or_assign(keys, sc, vals)
        check_against_model(t, model, dim)
        if with_assign:
            # raise some scores to the top of this batch's range: residents
            # stay resident, absent keys are ignored
            ak = rng.choice(pool, size=min(pool.size, 1 + batch // 3), replace=False)
            asc = u64(np.full(ak.size, _ASSIGN_TOP[scheme](step)))
            av = rng.standard_normal((ak.size, dim)).astype(np.float32)
            t.assign(ak, values=av, scores=asc)
            model.assign(ak, asc, av)
            check_against_model(t, model, dim)
        probe = rng.choice(pool, size=min(pool.size, 64), replace=False)
        got, found, fsc, _ = t.find(probe)
        res = model.resident_keys()
        for i, k in enumerate(probe.tolist()):
            assert bool(found[i]) == (k in res)
            if found[i]:
                assert int(fsc[i]) == model.score[k]
                np.testing.assert_array_equal(got[i], model.payload[k])


def test_single_bucket_adversarial_one_bucket():
    # every key routes to bucket 0 of a 4-bucket table
    t = oracle.OracleTable(capacity=4 * SLOTS, dim=2)
    rng = np.random.default_rng(5)
    cand = rand_keys(rng, 20000)
    keys = cand[t.route(cand)[0] == 0][:1500]
    model = TopKModel(lambda k: t.route(k)[0], 2)
    for step in range(1, 7):
        batch = rng.choice(keys, size=400, replace=False)
        sc = u64(step * 10 + rng.integers(0, 10, size=400))
        v = rng.standard_normal((400, 2)).astype(np.float32)
        t.insert_or_assign(batch, sc, values=v)
        model.insert_or_assign(batch, sc, v)
        check_against_model(t, model, 2)
    assert t.size() == SLOTS


def test_tiny_config_against_closed_form():
    """512 buckets x 128, dim 16, 8 batches of 16384 distinct keys drawn
    uniformly on [1, 2^40), score = batch index: exact per-bucket sets after
    every batch (every tie decided by (score, key))."""
    t = oracle.OracleTable(capacity=1 << 16, dim=16)
    model = TopKModel(lambda k: t.route(k)[0], 16)
    for step in range(1, 9):
        keys = gen.keys_in_range(0x484B560000000001, step, 16384, 1, 1 << 40).numpy().view(np.uint64)
        vals = gen.values(torch.from_numpy(keys.view(np.int64)), step, 16).numpy()
        sc = u64(np.full(16384, step))
        t.insert_or_assign(keys, sc, values=vals)
        model.insert_or_assign(keys, sc, vals)
        assert oracle_buckets(t) == model.resident()
    assert t.size() == model.size() == 1 << 16


def test_find_semantics_and_untouched_misses():
    rng = np.random.default_rng(9)
    t, model = random_workload(21, 8, 4, batches=6, batch=700, key_pool=3000, tie_heavy=False)
    res = model.resident_keys()
    seen = np.fromiter(model.score.keys(), dtype=np.uint64)
    absent = rand_keys(rng, 500)
    q = np.concatenate([seen, absent, u64([oracle.EMPTY_KEY, oracle.LOCKED_KEY])])
    sentinel = np.float32(-7.25)
    vals = np.full((q.size, 4), sentinel, np.float32)
    scores = np.full(q.size, 123456789, np.uint64)
    v, found, sc, _ = t.find(q, values_out=vals, scores_out=scores)
    for i, k in enumerate(q.tolist()):
        if k in res:
            assert found[i] == 1
            assert sc[i] == model.score[k]
            np.testing.assert_array_equal(v[i], model.payload[k])
        else:
            assert found[i] == 0
            assert sc[i] == 123456789
            assert (v[i] == sentinel).all()


def test_reserved_keys_are_skipped():
    t = oracle.OracleTable(capacity=SLOTS, dim=1)
    keys = u64([oracle.EMPTY_KEY, 5, oracle.LOCKED_KEY])
    out = t.insert_or_assign(keys, u64([1, 1, 1]), values=np.ones((3, 1), np.float32))
    assert out.tolist() == [oracle.SKIPPED, oracle.INSERTED, oracle.SKIPPED]
    assert t.size() == 1


def test_assign_updates_only_residents():
    rng = np.random.default_rng(3)
    t, model = random_workload(31, 4, 3, batches=5, batch=300, key_pool=1500, tie_heavy=False)
    before = oracle_buckets(t)
    seen = np.fromiter(model.score.keys(), dtype=np.uint64)
    keys = np.concatenate([rng.choice(seen, 400, replace=False), rand_keys(rng, 50)])
    newsc = u64(np.full(keys.size, 10 ** 9))
    newv = rng.standard_normal((keys.size, 3)).astype(np.float32)
    t.assign(keys, values=newv, scores=newsc)
    model.assign(keys, newsc, newv)
    assert oracle_buckets(t) == before  # structure unchanged (§3.5)
    check_against_model(t, model, 3)
    # score-only and value-only updates
    t.assign(keys[:10], scores=u64(np.full(10, 10 ** 9 + 1)))
    model.assign(keys[:10], scores=u64(np.full(10, 10 ** 9 + 1)))
    t.assign(keys[10:20], values=newv[:10] * 2)
    model.assign(keys[10:20], payload=newv[:10] * 2)
    check_against_model(t, model, 3)


def test_export_order_and_ranges():
    t, model = random_workload(41, 4, 2, batches=3, batch=200, key_pool=1000, tie_heavy=False)
    full = t.export()
    assert np.all(np.diff(full["pos"].astype(np.int64)) > 0)
    parts = [t.export(o, 100) for o in range(0, 4 * SLOTS, 100)]
    assert np.array_equal(np.concatenate([p["keys"] for p in parts]), full["keys"])
    assert t.export(4 * SLOTS, 10)["keys"].size == 0
    assert t.export(10, 0)["keys"].size == 0


def test_tag_mode_matches_value_mode():
    rng = np.random.default_rng(4)
    tv = oracle.OracleTable(capacity=4 * SLOTS, dim=2)
    tt = oracle.OracleTable(capacity=4 * SLOTS, dim=2, tag_mode=True)
    pool = rand_keys(rng, 2000)
    for step in range(1, 6):
        keys = rng.choice(pool, 500, replace=False)
        sc = u64(np.full(500, step))
        tags = u64(rng.integers(0, 1 << 62, 500))
        vals = np.stack([tags.astype(np.float32), -tags.astype(np.float32)], 1)
        o1 = tv.insert_or_assign(keys, sc, values=vals)
        o2 = tt.insert_or_assign(keys, sc, tags=tags)
        assert np.array_equal(o1, o2)
    a, b = tv.export(), tt.export()
    assert np.array_equal(a["keys"], b["keys"]) and np.array_equal(a["pos"], b["pos"])
    np.testing.assert_array_equal(a["values"][:, 0], b["tags"].astype(np.float32))


# ------------------------------------- find*, contains, insert_and_evict --

def test_find_pos_and_contains_match_layout():
    """find* reports where a resident key's row lives: its slot position (the
    row address is the value base plus that many rows, §3.6). Positions are
    checked against export (ascending positions, pinned above) and the key's
    routed bucket; found flags against the closed-form resident set."""
    rng = np.random.default_rng(12)
    t, model = random_workload(51, 8, 3, batches=6, batch=700, key_pool=3000, tie_heavy=True)
    res = model.resident_keys()
    e = t.export()
    where = dict(zip(e["keys"].tolist(), e["pos"].tolist()))
    seen = np.fromiter(model.score.keys(), dtype=np.uint64)
    q = np.concatenate([seen, rand_keys(rng, 300), u64([oracle.EMPTY_KEY, oracle.LOCKED_KEY])])
    found, pos = t.find_pos(q)
    b1 = t.route(q)[0]
    for i, k in enumerate(q.tolist()):
        if k in res:
            assert found[i] == 1 and int(pos[i]) == where[k] and int(pos[i]) // SLOTS == int(b1[i])
        else:
            assert found[i] == 0 and int(pos[i]) == 2 ** 64 - 1
    assert np.array_equal(t.contains(q), found)


def test_find_pos_dual_bucket_lands_in_a_candidate():
    rng = np.random.default_rng(13)
    t = oracle.OracleTable(capacity=8 * SLOTS, dim=1, dual=True)
    pool = rand_keys(rng, 4000)
    for step in range(1, 5):
        k = rng.choice(pool, 600, replace=False)
        t.insert_or_assign(k, u64(np.full(600, step)), values=np.zeros((600, 1), np.float32))
    e = t.export()
    found, pos = t.find_pos(e["keys"])
    assert found.all() and np.array_equal(pos, e["pos"])
    b1, b2, _ = t.route(e["keys"])
    assert np.all((pos // SLOTS == b1) | (pos // SLOTS == b2))


@pytest.mark.parametrize("tie_heavy", [False, True])
def test_insert_and_evict_returns_exactly_the_departed(tie_heavy):
    """Single-bucket mode: what insert_and_evict hands back is the entries that
    were resident before the call or offered by it and are not resident after
    it (closed form via the top-128 model), each with its last written value
    and score; the table itself ends as insert_or_assign would leave it."""
    rng = np.random.default_rng(14 + tie_heavy)
    B, dim = 4, 3
    t = oracle.OracleTable(capacity=B * SLOTS, dim=dim)
    model = TopKModel(lambda k: t.route(k)[0], dim)
    pool = rand_keys(rng, 3000)
    for step in range(1, 12):
        keys = rng.choice(pool, 400, replace=False)
        if tie_heavy:
            sc = u64(np.full(keys.size, step))
        else:
            sc = u64(step * 1000 + rng.integers(0, 1000, size=keys.size))
        vals = rng.standard_normal((keys.size, dim)).astype(np.float32)
        before = model.resident_keys()
        absent = sum(1 for k in keys.tolist() if k not in before)
        out = t.insert_and_evict(keys, sc, values=vals)
        model.insert_or_assign(keys, sc, vals)
        after = model.resident_keys()
        expect = (before | set(keys.tolist())) - after
        got = out["keys"].tolist()
        assert len(got) == len(set(got)) and set(got) == expect
        assert len(got) <= absent
        for k, s, v in zip(got, out["scores"].tolist(), out["values"]):
            assert model.score[k] == s
            np.testing.assert_array_equal(v, model.payload[k])
        check_against_model(t, model, dim)


def test_insert_and_evict_admission_bursts():
    """§5.4, Table 9 on a full table: a burst scored below every resident is
    handed back whole and changes nothing; a burst scored above every
    resident is admitted whole and hands back the lowest-ranked residents of
    each bucket it lands in."""
    C = 32 * SLOTS
    t = oracle.OracleTable(capacity=C, dim=1)
    stream = gen.unique_keys(6, 1, 0, 4 * C).numpy().view(np.uint64)
    i, step = 0, 10
    while t.size() < C:
        t.insert_or_assign(stream[i:i + 512], u64(np.full(512, step)), values=np.zeros((512, 1), np.float32))
        i += 512
        step += 1
    snap = t.export()
    low = gen.unique_keys(6, 2, 0, C // 8).numpy().view(np.uint64)
    out = t.insert_and_evict(low, u64(np.ones(low.size)), values=np.full((low.size, 1), 3.0, np.float32))
    assert sorted(out["keys"].tolist()) == sorted(low.tolist())
    assert np.all(out["scores"] == 1) and np.all(out["values"] == 3.0)
    after = t.export()
    assert np.array_equal(after["keys"], snap["keys"]) and np.array_equal(after["scores"], snap["scores"])
    high = gen.unique_keys(6, 3, 0, C // 8).numpy().view(np.uint64)
    out = t.insert_and_evict(high, u64(np.full(high.size, 10 ** 9)), values=np.zeros((high.size, 1), np.float32))
    assert out["keys"].size == high.size
    found, _ = t.find_pos(high)
    assert found.all()
    # per bucket, the handed-back residents are that bucket's lowest by (score, key)
    hb = t.route(high)[0]
    per_bucket = {}
    for b in hb.tolist():
        per_bucket[b] = per_bucket.get(b, 0) + 1
    snap_b = snap["pos"] // SLOTS
    expect = set()
    for b, c in per_bucket.items():
        m = snap_b == b
        order = np.lexsort((snap["keys"][m], snap["scores"][m]))
        expect |= set(snap["keys"][m][order][:c].tolist())
    assert set(out["keys"].tolist()) == expect


def test_find_or_insert_hits_and_inserts():
    """Hits: found = 1, the stored row comes back, the score becomes the offered
    one, the row is unchanged. Misses: inserted with the caller's row and score
    (insert_or_assign's admission), found = 0, the caller's row kept."""
    rng = np.random.default_rng(15)
    B, dim = 4, 2
    t = oracle.OracleTable(capacity=B * SLOTS, dim=dim)
    model = TopKModel(lambda k: t.route(k)[0], dim)
    pool = rand_keys(rng, 2500)
    for step in range(1, 10):
        keys = rng.choice(pool, 350, replace=False)
        sc = u64(np.full(keys.size, step))
        vals = rng.standard_normal((keys.size, dim)).astype(np.float32)
        before = model.resident_keys()
        rows, found = t.find_or_insert(keys, sc, values=vals)
        for i, k in enumerate(keys.tolist()):
            if k in before:
                assert found[i] == 1
                np.testing.assert_array_equal(rows[i], model.payload[k])
                model.score[k] = int(sc[i])
            else:
                assert found[i] == 0
                np.testing.assert_array_equal(rows[i], vals[i])
        miss = np.array([k not in before for k in keys.tolist()])
        model.insert_or_assign(keys[miss], sc[miss], vals[miss])
        check_against_model(t, model, dim)


@hypothesis.settings(max_examples=50, deadline=None, derandomize=True,
                     suppress_health_check=[hypothesis.HealthCheck.too_slow])
@hypothesis.given(
    seed=st.integers(0, 2**32 - 1),
    B=st.integers(1, 5),
    batches=st.integers(1, 6),
    batch=st.integers(1, 420),
    pool_factor=st.sampled_from([1, 2, 4]),
    scheme=st.sampled_from(["constant", "step", "coarse", "jitter"]),
    ops=st.lists(st.sampled_from(["insert_or_assign", "insert_and_evict", "find_or_insert"]), min_size=6,
                 max_size=6),
)
def test_inserters_closed_form_property(seed, B, batches, batch, pool_factor, scheme, ops):
    """Random tiny tables and batches, every inserter in random order: the
    table equals the top-128 model after each call (§3.1); insert_and_evict
    hands back exactly (resident before ∪ offered) − resident after with
    last-written rows and scores; find_or_insert flags exactly the keys
    resident before the call, returns their stored rows and refreshes their
    scores, and inserts the rest (§4.1)."""
    rng = np.random.default_rng(seed)
    dim = 2
    t = oracle.OracleTable(capacity=B * SLOTS, dim=dim)
    model = TopKModel(lambda k: t.route(k)[0], dim)
    pool = np.unique(rand_keys(rng, max(1, batch * pool_factor)))
    for step in range(1, batches + 1):
        keys = rng.choice(pool, size=min(batch, pool.size), replace=False)
        sc = _scores(scheme, rng, step, keys.size)
        vals = rng.standard_normal((keys.size, dim)).astype(np.float32)
        before = model.resident_keys()
        op = ops[step - 1]
        if op == "insert_or_assign":
            t.insert_or_assign(keys, sc, values=vals)
            model.insert_or_assign(keys, sc, vals)
        elif op == "insert_and_evict":
            out = t.insert_and_evict(keys, sc, values=vals)
            model.insert_or_assign(keys, sc, vals)
            after = model.resident_keys()
            got = out["keys"].tolist()
            assert len(got) == len(set(got)) and set(got) == (before | set(keys.tolist())) - after
            for k, s, v in zip(got, out["scores"].tolist(), out["values"]):
                assert model.score[k] == s
                np.testing.assert_array_equal(v, model.payload[k])
        else:
            rows, found = t.find_or_insert(keys, sc, values=vals)
            hit = np.array([k in before for k in keys.tolist()], dtype=bool)
            assert np.array_equal(found.astype(bool), hit)
            for i in np.flatnonzero(hit):
                np.testing.assert_array_equal(rows[i], model.payload[int(keys[i])])
                model.score[int(keys[i])] = int(sc[i])
            np.testing.assert_array_equal(rows[~hit], vals[~hit])
            model.insert_or_assign(keys[~hit], sc[~hit], vals[~hit])
        check_against_model(t, model, dim)


def test_new_operations_tag_mode_matches_value_mode():
    rng = np.random.default_rng(16)
    tv = oracle.OracleTable(capacity=4 * SLOTS, dim=2)
    tt = oracle.OracleTable(capacity=4 * SLOTS, dim=2, tag_mode=True)
    pool = rand_keys(rng, 2000)
    for step in range(1, 7):
        keys = rng.choice(pool, 500, replace=False)
        sc = u64(np.full(500, step))
        tags = u64(rng.integers(0, 1 << 24, 500))
        vals = np.stack([tags.astype(np.float32), -tags.astype(np.float32)], 1)
        if step % 2:
            a = tv.insert_and_evict(keys, sc, values=vals)
            b = tt.insert_and_evict(keys, sc, tags=tags)
            assert np.array_equal(a["keys"], b["keys"]) and np.array_equal(a["scores"], b["scores"])
            np.testing.assert_array_equal(a["values"][:, 0], b["tags"].astype(np.float32))
        else:
            ra, fa = tv.find_or_insert(keys, sc, values=vals)
            rb, fb = tt.find_or_insert(keys, sc, tags=tags)
            assert np.array_equal(fa, fb)
            np.testing.assert_array_equal(ra[:, 0], rb.astype(np.float32))
    a, b = tv.export(), tt.export()
    assert np.array_equal(a["keys"], b["keys"]) and np.array_equal(a["pos"], b["pos"])


# --------------------------------------------------------------- admission --

def test_admission_burst_low_and_high():
    """§5.4, Table 9 (scaled down): a table loaded to lambda = 0.96 with scores
    >= 10; a burst at score 1 evicts nobody (only empty slots may take burst
    keys); a burst at a score above every resident is admitted in full."""
    C = 64 * SLOTS
    t = oracle.OracleTable(capacity=C, dim=1)
    stream = gen.unique_keys(3, 1, 0, 4 * C).numpy().view(np.uint64)
    i = 0
    step = 10
    while t.size() < int(0.96 * C):
        n = min(512, int(0.96 * C) - t.size())
        k = stream[i:i + n]
        i += n
        t.insert_or_assign(k, u64(np.full(n, step)), values=np.zeros((n, 1), np.float32))
        step += 1
    before = set(t.export()["keys"].tolist())
    low = gen.unique_keys(3, 2, 0, C // 4).numpy().view(np.uint64)
    t.insert_or_assign(low, u64(np.ones(low.size)), values=np.zeros((low.size, 1), np.float32))
    after = set(t.export()["keys"].tolist())
    # No original displaced (hit-rate change zero). Burst keys may still take
    # empty slots and displace each other.
    assert before <= after
    high = gen.unique_keys(3, 3, 0, C // 4).numpy().view(np.uint64)
    out = t.insert_or_assign(high, u64(np.full(high.size, 10 ** 9)), values=np.zeros((high.size, 1), np.float32))
    assert np.all((out == oracle.EVICTED) | (out == oracle.INSERTED))
    _, found, _, _ = t.find(high)
    assert found.all()


# ------------------------------------------------------- Proposition 3.1 --

@pytest.mark.parametrize("lam", [0.5, 1.0])
def test_false_positive_compares_per_miss(lam):
    C = 512 * SLOTS
    t = oracle.OracleTable(capacity=C, dim=1)
    stream = gen.unique_keys(11, 1, 0, 3 * C).numpy().view(np.uint64)
    i = 0
    step = 1
    target = int(lam * C)
    while t.size() < target:
        n = min(8192, target - t.size()) if lam < 1 else 8192
        t.insert_or_assign(stream[i:i + n], u64(np.full(n, step)), values=np.zeros((n, 1), np.float32))
        i += n
        step += 1
    absent = gen.unique_keys(11, 2, 0, 200000).numpy().view(np.uint64)
    t.reset_probe_stats()
    _, found, _, _ = t.find(absent)
    assert found.sum() == 0
    probes, fp = t.probe_stats()
    assert probes == absent.size
    assert abs(fp / probes - 0.5) < 0.02  # S * 2^-8 = 0.5


# ------------------------------------------------------------ dual bucket --

def dual_keys(t, rng, n, distinct_buckets=True):
    cand = rand_keys(rng, 8 * n + 100)
    b1, b2, _ = t.route(cand)
    sel = cand[b1 != b2] if distinct_buckets else cand
    return sel[:n]


def test_dual_algorithm3_step_by_step():
    """Each key is applied alone and the state before/after is compared with
    Algorithm 3 restated on the union of the two candidate buckets: a present
    key is updated in place; with room in either bucket the key goes to the
    lowest empty slot of the less-occupied one (tie: the first); with both full
    the lowest (score, key) of the union is evicted iff the key ranks above it."""
    B = 6
    t = oracle.OracleTable(capacity=B * SLOTS, dim=1, dual=True)
    rng = np.random.default_rng(8)
    pool = rand_keys(rng, 3000)
    scores = {}
    for step in range(2500):
        k = int(rng.choice(pool))
        s = scores.get(k, 0) + int(rng.integers(0, 3))
        before = t.export()
        occ = np.bincount((before["pos"] // SLOTS).astype(np.int64), minlength=B)
        b1, b2, _ = (int(x[0]) for x in t.route(u64([k])))
        out = int(t.insert_or_assign(u64([k]), u64([s]), values=np.full((1, 1), step, np.float32))[0])
        after = t.export()
        bmap = dict(zip(before["keys"].tolist(), before["pos"].tolist()))
        amap = dict(zip(after["keys"].tolist(), after["pos"].tolist()))
        if k in bmap:
            assert out == oracle.UPDATED and amap[k] == bmap[k]
        elif occ[b1] < SLOTS or occ[b2] < SLOTS:
            tb = b1 if (b1 == b2 or occ[b1] <= occ[b2]) else b2
            assert out == oracle.INSERTED
            assert amap[k] == tb * SLOTS + occ[tb]
        else:
            union = [(sc, kk, p) for kk, sc, p in zip(before["keys"].tolist(), before["scores"].tolist(),
                                                    before["pos"].tolist()) if p // SLOTS in (b1, b2)]
            vs, vk, vp = min(union)
            if (s, k) > (vs, vk):
                assert out == oracle.EVICTED
                assert amap[k] == vp and vk not in amap
            else:
                assert out == oracle.REJECTED
                assert amap == bmap
        scores[k] = s
    assert t.size() <= B * SLOTS


def _evicted_score_mean(dual, trials, seed):
    rng = np.random.default_rng(seed)
    mins = []
    for _ in range(trials):
        t = oracle.OracleTable(capacity=2 * SLOTS, dim=1, dual=dual)
        keys = rand_keys(rng, 5000)
        b1, b2, _ = t.route(keys)
        # dual: only keys with two distinct candidates, so that phase D1 fills
        # both buckets without evicting (scores stay i.i.d.)
        pick = keys[b1 != b2] if dual else keys[b1 == 0]
        fill, newk = pick[:-1], pick[-1:]
        sc = u64(rng.integers(1, 1 << 63, size=fill.size)) * np.uint64(2)
        i = 0
        target = 2 * SLOTS if dual else SLOTS
        while t.size() < target:
            t.insert_or_assign(fill[i:i + 1], sc[i:i + 1], values=np.zeros((1, 1), np.float32))
            i += 1
        before = t.export()
        out = t.insert_or_assign(newk, u64([(1 << 64) - 1 - 1]), values=np.zeros((1, 1), np.float32))
        assert out[0] == oracle.EVICTED
        after = set(t.export()["keys"].tolist())
        gone = [s for k, s in zip(before["keys"].tolist(), before["scores"].tolist()) if k not in after]
        assert len(gone) == 1
        mins.append(gone[0] / 2.0 ** 64)
    return float(np.mean(mins))


def test_proposition_3_3_dual_halves_evicted_score():
    n = SLOTS
    single = _evicted_score_mean(False, 300, 1)
    dual = _evicted_score_mean(True, 300, 2)
    assert abs(single - 1 / (n + 1)) < 0.18 / (n + 1)
    assert abs(dual - 1 / (2 * n + 1)) < 0.18 / (2 * n + 1)


def _first_eviction_lambda(dual, seed):
    C = 1 << 20
    t = oracle.OracleTable(capacity=C, dim=1, dual=dual)
    keys = gen.unique_keys(seed, 1, 0, C).numpy().view(np.uint64)
    step = 0
    for i in range(0, C, 4096):
        step += 1
        k = keys[i:i + 4096]
        out = t.insert_or_assign(k, u64(np.full(k.size, step)), values=np.zeros((k.size, 1), np.float32))
        bad = np.nonzero((out == oracle.EVICTED) | (out == oracle.REJECTED))[0]
        if bad.size:
            return (i + int(bad[0])) / C  # every earlier key was inserted
    return 1.0


def test_first_eviction_load_factor_single_vs_dual():
    """§3.4: with 128-slot buckets a single-bucket table starts evicting well
    before it is full (birthday paradox), a dual-bucket table only near full.
    Single-mode band: the point where the expected number of buckets holding
    more than 128 of the keys reaches about one, for B = 8192 Poisson loads."""
    from scipy.stats import poisson

    B = (1 << 20) // SLOTS
    lam_grid = np.linspace(0.5, 1.0, 501)
    exp_over = [B * poisson.sf(SLOTS, SLOTS * l) for l in lam_grid]
    lam_pred = float(lam_grid[np.searchsorted(exp_over, 1.0)])
    single = _first_eviction_lambda(False, 5)
    dual = _first_eviction_lambda(True, 5)
    assert abs(single - lam_pred) < 0.06
    assert dual > 0.95 and dual > single + 0.15
