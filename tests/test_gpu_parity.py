"""Parity of the HIP table with the CPU oracle, through the C ABI.

Bar (everything here is integer/byte work, values are copied bit for bit):
* single-bucket mode: per-bucket contents equal as sets after every batch,
  size equal, find masks / values / scores bit-identical, rows and scores of
  misses untouched;
* serial insert mode (and dual-bucket serial mode): identical slot positions;
* dual-bucket parallel mode: invariants (no duplicate keys, occupancy <= 128,
  every resident entry carries its last write, found iff resident) plus top-N
  retention close to the oracle's.
"""

import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from conftest import gpu_available
from helpers import SLOTS, as_u64, group_by_bucket

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

NAN_BITS = 0x7FC00BAD  # a quiet NaN pattern that no generated value has
SENTINEL_SCORE = 0x5EED5EED5EED5EED


def dev():
    return torch.device("cuda", 0)


def hkv():
    import hash_table_cache_amd

    return hash_table_cache_amd


def np_u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def gpu_buckets(tab):
    k, _, _, p = tab.export_batch(with_values=False)
    return group_by_bucket(np_u64(k), np_u64(p))


def oracle_buckets(o):
    e = o.export()
    return group_by_bucket(e["keys"], e["pos"])


def assert_same_contents(tab, o, values=True):
    """Per-bucket key sets equal; every exported entry's score and row equal."""
    assert tab.size() == o.size()
    k, v, s, p = tab.export_batch(with_values=values)
    k, s, p = np_u64(k), np_u64(s), np_u64(p)
    assert np.unique(k).size == k.size
    assert group_by_bucket(k, p) == oracle_buckets(o)
    e = o.export()
    order_g = np.argsort(k)
    order_o = np.argsort(e["keys"])
    assert np.array_equal(k[order_g], e["keys"][order_o])
    assert np.array_equal(s[order_g], e["scores"][order_o])
    if values:
        vg = v.cpu().numpy()[order_g]
        vo = e["values"][order_o]
        assert np.array_equal(vg.view(np.uint32), vo.view(np.uint32))


def check_find(tab, o, q_keys, with_scores=True):
    """find on GPU vs oracle with NaN-prefilled rows and sentinel scores."""
    n = q_keys.numel()
    d = tab.dim
    vals = torch.full((n, d), 0, dtype=torch.int32, device=dev()).fill_(NAN_BITS).view(torch.float32)
    scores = torch.full((n,), SENTINEL_SCORE, dtype=torch.int64, device=dev()) if with_scores else None
    found = torch.full((n,), 7, dtype=torch.uint8, device=dev())
    tab.find(q_keys, values_out=vals, found_out=found, scores_out=scores)
    torch.cuda.synchronize()
    qk = np_u64(q_keys)
    ov = np.full((n, d), np.uint32(NAN_BITS).view(np.float32), np.float32)
    osc = np.full(n, SENTINEL_SCORE, np.uint64)
    _, ofound, osc, _ = o.find(qk, values_out=ov, scores_out=osc)
    assert np.array_equal(found.cpu().numpy(), ofound)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))
    if with_scores:
        assert np.array_equal(np_u64(scores), osc)
    return ofound


def sample_present(o, n, seed):
    e = o.export()
    rng = np.random.default_rng(seed)
    return rng.choice(e["keys"], size=min(n, e["keys"].size), replace=False)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(as_u64(a)).view(np.int64)).to(dev())


def mixed_queries(o, n, hit_frac, seed, absent_stream):
    nh = int(n * hit_frac)
    hits = sample_present(o, nh, seed)
    absent = gen.unique_keys(seed, absent_stream, 0, n - hits.size).numpy().view(np.uint64)
    q = np.concatenate([hits, absent])
    q = np.random.default_rng(seed + 1).permutation(q)
    return to_dev(q)


# ------------------------------------------------------------------------------

def test_tiny_single_bucket_workload_exact():
    """512 buckets x 128 slots, dim 16, 8 upsert batches of 16384 distinct keys
    uniform on [1, 2^40) with score = batch index (lambda reaches 1.0), then a
    find of 16384 keys, half resident, half absent."""
    H = hkv()
    C, D = 1 << 16, 16
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    seed = 0x484B560000000001
    for step in range(1, 9):
        keys = gen.keys_in_range(seed, step, 16384, 1, 1 << 40, device=dev())
        vals = gen.values(keys, step, D)
        sc = torch.full((16384,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
        assert_same_contents(tab, o)
    assert tab.size() == C
    q = mixed_queries(o, 16384, 0.5, seed, 99)
    found = check_find(tab, o, q)
    assert found.sum() == 8192


@pytest.mark.parametrize("lam,unique_keys", [(0.5, False), (0.75, False), (0.9, False), (1.0, False), (1.0, True)])
def test_lambda_sweep_reduced_exact(lam, unique_keys):
    """Load-factor sweep at reduced capacity (2^20 slots, dim 32, batches of
    2^16 distinct uniform keys, score = batch index), then find with 90 % hits."""
    H = hkv()
    C, D, nb = 1 << 20, 32, 1 << 16
    tab = H.HashTable(C, D, unique_keys=unique_keys)
    o = oracle.OracleTable(C, D)
    target = int(round(lam * C))
    step, start = 0, 0
    while True:
        size = o.size()
        if size >= target:
            break
        n = nb if lam >= 1.0 else min(nb, target - size)
        step += 1
        keys = gen.unique_keys(20 + int(lam * 100), 1, start, n, device=dev())
        start += n
        vals = gen.values(keys, step, D)
        sc = torch.full((n,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
    assert_same_contents(tab, o)
    q = mixed_queries(o, 1 << 16, 0.9, 5, 77)
    check_find(tab, o, q)


def one_new_key_per_bucket(o, seed, stream, start, buckets):
    """One never-inserted key routed to each of `buckets` distinct buckets
    (drawn from a unique-key stream; returns the keys and the next cursor)."""
    picked = {}
    cur = start
    while len(picked) < buckets:
        cand = np_u64(gen.unique_keys(seed, stream, cur, 4 * buckets))
        cur += 4 * buckets
        b1, _, _ = o.route(cand)
        for k, b in zip(cand.tolist(), b1.tolist()):
            if b not in picked:
                picked[b] = k
    keys = np.array([picked[b] for b in sorted(picked)], dtype=np.uint64)
    return torch.from_numpy(keys.view(np.int64)).to(dev()), cur


@pytest.mark.parametrize("resident_scores", ["all_equal", "spread"])
def test_single_new_key_per_full_bucket_exact(resident_scores):
    """Every batch sends exactly one new key to each bucket of a full table,
    so each bucket's chain is that one key and its owner decides eviction
    from the score column and the keys tied at the lowest score. Residents
    all share one score ("all_equal": every slot is tied) or carry spread
    scores with a few ties ("spread"); the new keys' scores equal the lowest
    resident score in half of the batches (admitted iff the key outranks the
    lowest key) and exceed it in the others. Contents match the oracle after
    every batch."""
    H = hkv()
    C, D = 1 << 14, 16
    nbk = C // SLOTS
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    seed = 0x484B56000000F11E
    cur = 0
    step = 0
    while o.size() < C:
        step += 1
        n = C
        keys = gen.unique_keys(seed, 1, cur, n, device=dev())
        cur += n
        if resident_scores == "all_equal":
            sc = torch.full((n,), 100, dtype=torch.int64, device=dev())
        else:
            sc = 100 + (gen.counter_words(seed, 2, cur, n, dev()) & 7)  # 8 score levels, many ties
        vals = gen.values(keys, step, D)
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
    assert_same_contents(tab, o)
    ncur = 0
    for j in range(6):
        step += 1
        keys, ncur = one_new_key_per_bucket(o, seed, 3, ncur, nbk)
        lowest = int(o.export()["scores"].min())
        base = lowest if j % 2 == 0 else lowest + 1
        sc = torch.full((keys.numel(),), base, dtype=torch.int64, device=dev())
        vals = gen.values(keys, step, D)
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
        assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 4096, 0.5, seed, 9))


@pytest.mark.parametrize("unique_keys", [False, True])
def test_mixed_find_assign_upsert_reduced_exact(unique_keys):
    """Reader / updater / inserter steps at lambda = 1 (2^17 slots, dim 64):
    per step a find, an assign of resident keys, an upsert of half fresh and
    half resident keys; exact after every step. Also on a table created with
    the distinct-keys promise (no per-slot claims on in-place updates)."""
    H = hkv()
    C, D = 1 << 17, 64
    tab = H.HashTable(C, D, unique_keys=unique_keys)
    o = oracle.OracleTable(C, D)
    step, start = 0, 0
    while o.size() < C:
        step += 1
        keys = gen.unique_keys(31, 1, start, 1 << 14, device=dev())
        start += 1 << 14
        vals = gen.values(keys, step, D)
        sc = torch.full((keys.numel(),), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
    assert_same_contents(tab, o)
    for t in range(4):
        step += 1
        q = mixed_queries(o, 1 << 14, 0.9, 100 + t, 200 + t)
        check_find(tab, o, q)
        ak = to_dev(sample_present(o, 1 << 13, 300 + t))
        av = gen.values(ak, step * 2, D)
        asc = torch.full((ak.numel(),), step, dtype=torch.int64, device=dev())
        tab.assign(ak, av, asc)
        o.assign(np_u64(ak), values=av.cpu().numpy(), scores=np_u64(asc))
        fresh = gen.unique_keys(31, 2, t * 4096, 4096).numpy().view(np.uint64)
        old = sample_present(o, 4096, 400 + t)
        uk = to_dev(np.random.default_rng(t).permutation(np.concatenate([fresh, old])))
        uv = gen.values(uk, step * 2 + 1, D)
        usc = torch.full((uk.numel(),), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(uk, uv, usc)
        o.insert_or_assign(np_u64(uk), np_u64(usc), values=uv.cpu().numpy())
        assert_same_contents(tab, o)


def test_batch_order_does_not_change_contents():
    """Single-bucket contents after a batch are the same for any in-batch
    order (serializable per bucket, monotone scores)."""
    H = hkv()
    C, D = 1 << 14, 4
    base = gen.unique_keys(5, 1, 0, 3 * C, device=dev())
    sets = []
    for perm_seed in range(3):
        tab = H.HashTable(C, D)
        for step in range(3):
            k = base[step * C:(step + 1) * C]
            k = gen.shuffle(k, perm_seed, step)
            sc = (k & 3) + step * 10  # a function of the key: the same in every order
            tab.insert_or_assign(k, gen.values(k, step, D), sc)
        sets.append(gpu_buckets(tab))
        tab.close()
    assert sets[0] == sets[1] == sets[2]


@pytest.mark.parametrize("dual", [False, True])
def test_serial_insert_mode_identical_positions(dual):
    """With serial inserts the GPU applies keys in input order and must place
    every key in exactly the oracle's slot (Algorithms 2 and 3)."""
    H = hkv()
    C, D = 16 * SLOTS, 3
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=dual)
    rng = np.random.default_rng(6)
    pool = rng.integers(1, 1 << 62, size=5000, dtype=np.int64)
    for step in range(1, 12):
        k = np.unique(rng.choice(pool, 600, replace=False))
        k = rng.permutation(k)
        kt = torch.from_numpy(k).to(dev())
        sc = torch.from_numpy(step * 4 + rng.integers(0, 4, size=k.size)).to(dev())
        v = gen.values(kt, step, D)
        tab.insert_or_assign(kt, v, sc)
        o.insert_or_assign(k.view(np.uint64), np_u64(sc), values=v.cpu().numpy())
        gk, _, gs, gp = tab.export_batch(with_values=False)
        e = o.export()
        order = np.argsort(np_u64(gp))
        assert np.array_equal(np_u64(gp)[order], e["pos"])
        assert np.array_equal(np_u64(gk)[order], e["keys"])
        assert np.array_equal(np_u64(gs)[order], e["scores"])
    assert_same_contents(tab, o)


def test_dual_serial_zipf_lfu_stream_identical_positions():
    """Serial dual-bucket mode under the online workload's shape, scaled
    down: 256 buckets, batches of 16384 Zipf(1.05) draws over 2^20 ids,
    deduplicated, score = cumulative frequency (ties everywhere at the low
    end), driven well past full capacity so that D2 (the lower recorded
    minimum, ties by key) decides most inserts. Every key's slot, score and
    row equal the oracle's (Algorithm 3 applied key by key) after every
    batch."""
    H = hkv()
    C, D = 256 * SLOTS, 2
    tab = H.HashTable(C, D, dual_bucket=True, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=True)
    zipf = gen.Zipf(1.05, 1 << 20)
    freq = torch.zeros((1 << 20) + 1, dtype=torch.int64, device=dev())
    full_at = None
    for b in range(40):
        r = zipf.draw(0x5EED0D2, 1, b * 16384, 16384, device=dev())
        uniq, cnt = torch.unique(r, return_counts=True)
        freq.index_add_(0, uniq, cnt)
        sc = freq[uniq]
        perm = torch.from_numpy(np.random.default_rng(b).permutation(uniq.numel())).to(dev())
        k, s2 = uniq[perm].contiguous(), sc[perm].contiguous()
        v = gen.values(k, s2, D)
        tab.insert_or_assign(k, v, s2)
        o.insert_or_assign(np_u64(k), np_u64(s2), values=v.cpu().numpy())
        gk, _, gs, gp = tab.export_batch(with_values=False)
        e = o.export()
        order = np.argsort(np_u64(gp))
        assert np.array_equal(np_u64(gp)[order], e["pos"]), f"batch {b}"
        assert np.array_equal(np_u64(gk)[order], e["keys"]), f"batch {b}"
        assert np.array_equal(np_u64(gs)[order], e["scores"]), f"batch {b}"
        if full_at is None and e["keys"].size == C:
            full_at = b
    assert full_at is not None and full_at < 10, "the stream should fill the table early"
    assert_same_contents(tab, o)


def test_adversarial_all_keys_one_bucket():
    H = hkv()
    C, D = 8 * SLOTS, 8
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    cand = np.random.default_rng(2).integers(1, 1 << 62, size=40000, dtype=np.int64).view(np.uint64)
    keys = cand[o.route(cand)[0] == 3][:2000]
    for step in range(1, 4):
        k = to_dev(keys[(step - 1) * 600: step * 600 + 100])
        sc = torch.full((k.numel(),), step, dtype=torch.int64, device=dev())
        v = gen.values(k, step, D)
        tab.insert_or_assign(k, v, sc)
        o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
        assert_same_contents(tab, o)
    check_find(tab, o, to_dev(keys))


@pytest.mark.parametrize("hot_buckets", [1, 2, 4])
def test_contention_few_buckets_mixed_with_updates(hot_buckets):
    """Contention stress: every key of each batch routes to one of 1, 2 or 4
    buckets of a 64-bucket table, batches mix new keys with updates of
    resident ones and with keys that lose admission, and the scores jitter
    within a step (ties broken by key). Contents exact after every batch,
    and insert_and_evict's hand-back exact on the same stream."""
    H = hkv()
    C, D = 64 * SLOTS, 4
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    rng = np.random.default_rng(40 + hot_buckets)
    cand = rng.integers(1, 1 << 62, size=400000, dtype=np.int64).view(np.uint64)
    b1 = o.route(cand)[0]
    hot = rng.choice(64, size=hot_buckets, replace=False)
    keys = cand[np.isin(b1, hot)][:3000]
    resident = []
    for step in range(1, 9):
        fresh = keys[(step - 1) * 300: step * 300]
        old = rng.choice(np.array(resident, dtype=np.uint64), size=min(200, len(resident)), replace=False) \
            if resident else np.zeros(0, np.uint64)
        k = rng.permutation(np.concatenate([fresh, old]))
        sc = (step * 4 + rng.integers(0, 4, size=k.size)).astype(np.uint64)
        kt, st = to_dev(k), to_dev(sc)
        v = gen.values(kt, step, D)
        if step % 2:
            tab.insert_or_assign(kt, v, st)
            o.insert_or_assign(k, sc, values=v.cpu().numpy())
        else:
            ek, ev, es, cnt = tab.insert_and_evict(kt, v, st)
            want = o.insert_and_evict(k, sc, values=v.cpu().numpy())
            torch.cuda.synchronize()
            m = int(cnt.item())
            order = np.argsort(np_u64(ek[:m]))
            wo = np.argsort(want["keys"])
            assert np.array_equal(np_u64(ek[:m])[order], want["keys"][wo])
            assert np.array_equal(np_u64(es[:m])[order], want["scores"][wo])
            assert np.array_equal(ev[:m].cpu().numpy()[order].view(np.uint32), want["values"][wo].view(np.uint32))
        assert_same_contents(tab, o)
        resident = o.export()["keys"].tolist()
    check_find(tab, o, to_dev(keys[:2400]))


def test_inserter_epoch_wrap_keeps_chains_exact(monkeypatch):
    """Chain heads carry the inserter call's epoch and are never reset; the
    per-table call counter starts just below its wrap here, so the calls run
    at epochs 2^32-2, 2^32-1, then (heads reset) 1, 2, ... Every batch sends
    many keys to the same few buckets (long chains, heads left by the
    previous call in every one of them); contents exact after each call."""
    monkeypatch.setenv("HKV_EPOCH_START", str(0xFFFFFFFD))
    H = hkv()
    C, D = 16 * SLOTS, 8
    tab = H.HashTable(C, D)
    monkeypatch.delenv("HKV_EPOCH_START")
    o = oracle.OracleTable(C, D)
    rng = np.random.default_rng(77)
    cand = rng.integers(1, 1 << 62, size=200000, dtype=np.int64).view(np.uint64)
    keys = cand[np.isin(o.route(cand)[0], [2, 5, 11])][:2400]
    for step in range(1, 7):
        k = keys[(step - 1) * 400: step * 400]
        sc = (step * 2 + rng.integers(0, 2, size=k.size)).astype(np.uint64)
        kt, st = to_dev(k), to_dev(sc)
        v = gen.values(kt, step, D)
        if step == 4:
            f, _ = tab.find_or_insert(kt, v, st)
            o.find_or_insert(k, sc, values=v.cpu().numpy())
        else:
            tab.insert_or_assign(kt, v, st)
            o.insert_or_assign(k, sc, values=v.cpu().numpy())
        assert_same_contents(tab, o)
    check_find(tab, o, to_dev(keys))


def test_edge_cases_reserved_empty_duplicates():
    H = hkv()
    C, D = 4 * SLOTS, 4
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    empty = torch.empty(0, dtype=torch.int64, device=dev())
    tab.insert_or_assign(empty, torch.empty((0, D), device=dev()), empty)
    tab.find(empty)
    tab.assign(empty, scores=empty)
    assert tab.size() == 0
    special = as_u64([oracle.EMPTY_KEY, oracle.LOCKED_KEY, 1, 2, 3])
    k = to_dev(special)
    v = gen.values(k, 1, D)
    sc = torch.ones(5, dtype=torch.int64, device=dev())
    tab.insert_or_assign(k, v, sc)
    o.insert_or_assign(special, np_u64(sc), values=v.cpu().numpy())
    assert tab.size() == 3
    tab.assign(k, scores=sc * 5)
    o.assign(special, scores=np_u64(sc * 5))
    assert_same_contents(tab, o)
    # duplicate queries are fine for readers
    q = to_dev(as_u64([1, 1, 2, oracle.EMPTY_KEY, 9, 2]))
    check_find(tab, o, q)
    # empty export ranges
    kk, _, _, _ = tab.export_batch(offset=C, n_slots=10)
    assert kk.numel() == 0


@pytest.mark.parametrize("D", [1, 3, 5, 8, 33])
def test_odd_dims_and_unaligned_rows(D):
    """dim not a multiple of 4 and outputs that are not 16-byte aligned take
    the scalar copy path; results stay exact."""
    H = hkv()
    C = 8 * SLOTS
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    for step in range(1, 4):
        k = gen.unique_keys(8, 1, (step - 1) * 700, 700, device=dev())
        v = gen.values(k, step, D)
        sc = torch.full((700,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(k, v, sc)
        o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
    assert_same_contents(tab, o)
    q = mixed_queries(o, 500, 0.6, 3, 9)
    check_find(tab, o, q)
    # unaligned output rows: a view starting one float into a buffer
    buf = torch.zeros(500 * D + 1, dtype=torch.float32, device=dev())
    out = buf[1:].view(500, D)
    found = torch.empty(500, dtype=torch.uint8, device=dev())
    tab.find(q, values_out=out, found_out=found)
    ref_v, ref_f, _, _ = o.find(np_u64(q))
    f = found.cpu().numpy().astype(bool)
    assert np.array_equal(f, ref_f.astype(bool))
    assert np.array_equal(out.cpu().numpy()[f].view(np.uint32), ref_v[f].view(np.uint32))


def test_non_power_of_two_bucket_count():
    H = hkv()
    C, D = 6 * SLOTS, 4
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    for step in range(1, 5):
        k = gen.unique_keys(12, 1, (step - 1) * 500, 500, device=dev())
        v = gen.values(k, step, D)
        sc = torch.full((500,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(k, v, sc)
        o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
        assert_same_contents(tab, o)


def test_values_on_host_tiered_mode():
    """Value rows in pinned host memory mapped into the GPU (§3.6)."""
    H = hkv()
    C, D = 64 * SLOTS, 32
    tab = H.HashTable(C, D, values_on_host=True)
    o = oracle.OracleTable(C, D)
    for step in range(1, 4):
        k = gen.unique_keys(13, 1, (step - 1) * 4000, 4000, device=dev())
        v = gen.values(k, step, D)
        sc = torch.full((4000,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(k, v, sc)
        o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
    assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 3000, 0.9, 4, 5))
    ak = to_dev(sample_present(o, 1000, 6))
    av = gen.values(ak, 99, D)
    tab.assign(ak, av)
    o.assign(np_u64(ak), values=av.cpu().numpy())
    assert_same_contents(tab, o)


def test_export_then_reinsert_restores_the_table():
    """Checkpoint and resume through the public calls: export a full table
    (after evictions) in slot ranges, destroy it, insert the exported keys,
    rows and scores into a new table in shuffled order. Every bucket held at
    most 128 entries, all routed to it, so the new table has the same
    per-bucket sets, rows and scores as the oracle that followed the first."""
    H = hkv()
    C, D = 48 * SLOTS, 16
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    seed = 0x484B5600000C4EC7
    for step in range(1, 5):
        keys = gen.unique_keys(seed, 1, (step - 1) * 3000, 3000, device=dev())
        sc = 10 * step + (gen.counter_words(seed, 2, step * 3000, 3000, dev()) & 7)
        vals = gen.values(keys, step, D)
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
    assert tab.size() == C
    parts = [tab.export_batch(off, 1000) for off in range(0, C, 1000)]
    k = torch.cat([q[0] for q in parts])
    v = torch.cat([q[1] for q in parts])
    s_ = torch.cat([q[2] for q in parts])
    tab.close()
    assert k.numel() == C
    order = torch.from_numpy(np.random.default_rng(5).permutation(C)).to(dev())
    k, v, s_ = k[order].contiguous(), v[order].contiguous(), s_[order].contiguous()
    fresh = H.HashTable(C, D)
    fresh.insert_or_assign(k, v, s_)
    assert_same_contents(fresh, o)
    check_find(fresh, o, mixed_queries(o, 5000, 0.8, seed, 3))
    fresh.close()


def test_export_ranges_partition_the_table():
    H = hkv()
    C, D = 16 * SLOTS, 2
    tab = H.HashTable(C, D)
    k = gen.unique_keys(14, 1, 0, 1500, device=dev())
    tab.insert_or_assign(k, gen.values(k, 1, D), torch.ones(1500, dtype=torch.int64, device=dev()))
    whole = set(np_u64(tab.export_batch()[0]).tolist())
    parts = set()
    for off in range(0, C, 300):
        kk, _, _, pp = tab.export_batch(off, 300, with_values=False)
        pos = np_u64(pp)
        assert np.all((pos >= off) & (pos < off + 300))
        parts |= set(np_u64(kk).tolist())
    assert parts == whole and len(whole) == tab.size()


def test_allocation_failure_is_reported_and_leaves_the_device_usable():
    """A table whose rows cannot fit in HBM (2^20 slots of 2^20 floats: 4 TiB)
    fails with HKV_ENOMEM and frees what it had allocated; a normal table
    created right after works."""
    H = hkv()
    with pytest.raises(H.HkvError) as ei:
        H.HashTable(1 << 20, 1 << 20)
    assert ei.value.status == -2
    assert "capacity" in str(ei.value)
    tab = H.HashTable(4 * SLOTS, 8)
    k = torch.arange(1, 301, dtype=torch.int64, device=dev())
    tab.insert_or_assign(k, gen.values(k, 1, 8), torch.ones(300, dtype=torch.int64, device=dev()))
    _, found, _ = tab.find(k)
    torch.cuda.synchronize()
    assert int(found.sum()) == min(300, tab.size()) and tab.size() > 0
    tab.close()


def test_invalid_pointers_are_rejected():
    H = hkv()
    tab = H.HashTable(SLOTS, 4)
    k = torch.arange(10, dtype=torch.int64)  # pageable host memory
    with pytest.raises(H.HkvError) as ei:
        tab.find(k, values_out=torch.zeros((10, 4)), found_out=torch.zeros(10, dtype=torch.uint8))
    assert ei.value.status == -1
    kd = torch.arange(10, dtype=torch.int64, device=dev())
    with pytest.raises(H.HkvError):
        tab.assign(kd)  # neither values nor scores
    small = torch.zeros((5, 4), device=dev())
    from hash_table_cache_amd import _native

    with pytest.raises(ValueError):
        _native.hkv_find(tab.handle, kd, small, torch.zeros(10, dtype=torch.uint8, device=dev()),
                         dim=4, device=0)


def test_batches_beyond_the_index_limit_are_refused():
    """Batch indices 2^32 - 4 .. 2^32 - 1 mark chain ends in the inserter, so
    every batched call refuses n > 2^32 - 4 with HKV_EINVAL, before it reads
    any buffer (the pointers here are small device buffers, never touched)."""
    from hash_table_cache_amd import _native

    H = hkv()
    L = _native.load()
    tab = H.HashTable(SLOTS, 4)
    h = tab.handle
    buf = torch.zeros(64, dtype=torch.int64, device=dev())
    p = buf.data_ptr()
    n = (1 << 32) - 3
    calls = {
        "find": lambda: L.hkv_find(h, n, p, p, p, None, None),
        "find_ptr": lambda: L.hkv_find_ptr(h, n, p, p, p, None, None),
        "contains": lambda: L.hkv_contains(h, n, p, p, None),
        "insert_or_assign": lambda: L.hkv_insert_or_assign(h, n, p, p, p, None),
        "insert_and_evict": lambda: L.hkv_insert_and_evict(h, n, p, p, p, p, None, None, p, None),
        "find_or_insert": lambda: L.hkv_find_or_insert(h, n, p, p, p, None, None),
        "assign": lambda: L.hkv_assign(h, n, p, p, p, None),
    }
    for name, c in calls.items():
        assert c() == _native.HKV_EINVAL, name
        assert b"exceeds the limit" in L.hkv_last_error(), name
    assert tab.size() == 0
    tab.close()


def test_group_ordering_across_streams():
    """An upsert on one stream followed, without host synchronization, by a
    find on another stream must observe the upsert: the library orders the
    reader after the inserter (§3.5, Table 4)."""
    H = hkv()
    C, D = 1 << 16, 16
    tab = H.HashTable(C, D)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    n = 20000
    keys = [gen.unique_keys(15, 1 + r, 0, n, device=dev()) for r in range(2)]
    vals = [gen.values(k, 1, D) for k in keys]
    sc = torch.ones(n, dtype=torch.int64, device=dev())
    outs = [torch.zeros((n, D), device=dev()) for _ in range(2)]
    founds = [torch.zeros(n, dtype=torch.uint8, device=dev()) for _ in range(2)]
    torch.cuda.synchronize()
    for r in range(2):
        tab.insert_or_assign(keys[r], vals[r], sc, stream=s1)
        tab.find(keys[r], values_out=outs[r], found_out=founds[r], stream=s2)
    torch.cuda.synchronize()
    for r in range(2):
        assert int(founds[r].sum()) == n  # at most ~80 keys per bucket: nothing evicted
        assert torch.equal(outs[r], vals[r])


def test_dual_bucket_invariants_and_retention():
    """Dual-bucket parallel inserts under a Zipf stream with frequency scores:
    invariants after every batch, and top-N retention close to the oracle's."""
    H = hkv()
    C, D = 1 << 15, 8
    tab = H.HashTable(C, D, dual_bucket=True)
    o = oracle.OracleTable(C, D, dual=True, tag_mode=True)
    z = gen.Zipf(1.05, 1 << 20)
    freq = {}
    for b in range(24):
        r = z.draw(77, 1, b * 8192, 8192).numpy()
        uniq, cnt = np.unique(r, return_counts=True)
        for x, c in zip(uniq.tolist(), cnt.tolist()):
            freq[x] = freq.get(x, 0) + c
        keys = uniq.astype(np.uint64)
        sc = np.array([freq[x] for x in uniq.tolist()], dtype=np.uint64)
        kt = to_dev(keys)
        st = to_dev(sc)
        v = gen.values(kt, st, D)
        tab.insert_or_assign(kt, v, st)
        o.insert_or_assign(keys, sc, tags=sc)
        gk, gv, gs, gp = tab.export_batch()
        k_, s_, p_ = np_u64(gk), np_u64(gs), np_u64(gp)
        assert np.unique(k_).size == k_.size
        assert tab.size() == k_.size <= C
        assert np.bincount((p_ // SLOTS).astype(np.int64)).max() <= SLOTS
        assert all(freq[x] == s for x, s in zip(k_.tolist(), s_.tolist()))
        assert torch.equal(gv, gen.values(gk, gs, D))
        b1, b2, _ = o.route(k_)
        assert np.all((p_ // SLOTS == b1) | (p_ // SLOTS == b2))
    # top-N retention against the ideal top-N by (frequency, key)
    allk = np.array(sorted(freq, key=lambda x: (freq[x], x), reverse=True)[:C], dtype=np.uint64)
    ideal = set(allk.tolist())
    gpu_ret = len(ideal & set(k_.tolist())) / C
    ora_ret = len(ideal & set(o.export()["keys"].tolist())) / C
    assert gpu_ret > ora_ret - 0.01
    q = to_dev(np.array(list(freq.keys()), dtype=np.uint64)[:20000])
    vals, found, scs = tab.find(q, with_scores=True)
    res = set(k_.tolist())
    qn = np_u64(q)
    f = found.cpu().numpy().astype(bool)
    assert np.array_equal(f, np.array([x in res for x in qn.tolist()]))
    assert all(freq[x] == s for x, s in zip(qn[f].tolist(), np_u64(scs)[f].tolist()))


@pytest.mark.parametrize("dual,unique_keys", [(False, False), (True, False), (False, True)])
def test_duplicate_keys_in_a_batch_keep_the_table_consistent(dual, unique_keys):
    """Duplicates within one write batch: which occurrence wins is unspecified,
    but no key may become resident twice and every stored row must be one of
    the rows written for that key (full buckets, so evictions happen too).
    The key-level part holds even on a table whose caller promised distinct
    keys and broke the promise."""
    H = hkv()
    C, D = 32 * SLOTS, 4
    tab = H.HashTable(C, D, dual_bucket=dual, unique_keys=unique_keys)
    rng = np.random.default_rng(17)
    pool = rng.integers(1, 1 << 62, size=3 * C, dtype=np.int64)
    written = {}
    for step in range(1, 9):
        base = rng.choice(pool, size=C // 2, replace=False)
        k = np.concatenate([base, rng.choice(base, size=C // 4)])  # ~1/3 duplicated
        k = rng.permutation(k)
        kt = torch.from_numpy(k).to(dev())
        ver = torch.arange(k.size, dtype=torch.int64, device=dev()) + step * 100000
        v = gen.values(kt, ver, D)
        sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(kt, v, sc)
        for kk, vv in zip(k.view(np.uint64).tolist(), ver.cpu().numpy().tolist()):
            written.setdefault(kk, set()).add(vv)
        gk, gv, gs, gp = tab.export_batch()
        ku = np_u64(gk)
        assert np.unique(ku).size == ku.size
        assert tab.size() == ku.size <= C
        # each resident row is the row of one of the versions written for that key
        gvn = gv.cpu().numpy()
        for j in rng.choice(ku.size, size=min(200, ku.size), replace=False).tolist():
            key = int(ku[j])
            vers = torch.tensor(sorted(written[key]), dtype=torch.int64)
            cand = gen.values(torch.full((vers.numel(),), int(np.uint64(key).view(np.int64)), dtype=torch.int64),
                              vers, D).numpy()
            assert any(np.array_equal(cand[r].view(np.uint32), gvn[j].view(np.uint32)) for r in range(len(vers)))


@pytest.mark.parametrize("dual", [False, True])
def test_duplicate_keys_store_one_occurrence_whole(dual):
    """Each key of a write batch occurring many times, dim 64 (16 lanes'
    worth of 16-byte pieces per row), every occurrence with its own row and
    score: afterwards each key is resident once and its stored (row, score)
    is exactly one occurrence's pair, whole, for resident keys updated in
    place and for new keys alike. Checked on every touched key."""
    H = hkv()
    C, D = 1 << 15, 64
    tab = H.HashTable(C, D, dual_bucket=dual)
    rng = np.random.default_rng(23)
    # half full: no key leaves, so every touched key stays resident
    base = gen.unique_keys(23, 1, 0, C // 2, device=dev())
    tab.insert_or_assign(base, gen.values(base, 1, D), torch.ones(base.numel(), dtype=torch.int64, device=dev()))
    fresh_pool = gen.unique_keys(23, 2, 0, 4096, device=dev())
    for step in range(2, 6):
        res = base[torch.from_numpy(rng.choice(base.numel(), size=2048, replace=False)).to(dev())]
        new = fresh_pool[(step - 2) * 256:(step - 1) * 256]
        k = torch.cat([res.repeat(8), new.repeat(8)])
        k = k[torch.from_numpy(rng.permutation(k.numel())).to(dev())]
        ver = torch.arange(k.numel(), dtype=torch.int64, device=dev()) + step * 1_000_000
        tab.insert_or_assign(k, gen.values(k, ver, D), ver)
        gk, gv, gs, gp = tab.export_batch()
        assert torch.unique(gk).numel() == gk.numel()
        assert tab.size() == gk.numel() == base.numel() + (step - 1) * 256
        touched = torch.unique(k)
        pos = torch.searchsorted(torch.sort(gk).values, touched)
        order = torch.argsort(gk)
        sk, sv, ss = gk[order], gv[order], gs[order]
        assert torch.equal(sk[pos], touched), "a touched key is not resident"
        s = ss[pos]
        # the stored score is one of this key's occurrences' (versions are
        # distinct and ascending, one per occurrence) ...
        idx = torch.clamp(torch.searchsorted(ver, s), max=ver.numel() - 1)
        assert torch.equal(ver[idx], s)
        assert torch.equal(k[idx], touched), "stored score belongs to another key's occurrence"
        # ... and the stored row is that same occurrence's row, whole
        assert torch.equal(sv[pos].view(torch.int32), gen.values(touched, s, D).view(torch.int32)), \
            "a stored row mixes occurrences"
    tab.close()
