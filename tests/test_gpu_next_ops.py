"""Parity of find*, contains, insert_and_evict and find_or_insert (the
cache-specific calls of the paper's §4.1) with the CPU oracle, through the C ABI.

Bar: found flags, scores and rows bit-exact; find* addresses equal to one
value base plus the slot position times the row size, with the positions of
export (and, in serial mode, of the oracle); insert_and_evict's hand-back
equal to the oracle's as a set of (key, score, row) in single-bucket mode and
in identical order in serial mode; table contents equal after every call.
Dual-bucket parallel mode: the hand-back and the table together hold exactly
what was resident or offered, nothing twice.
"""

import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from conftest import gpu_available
from helpers import SLOTS
from test_gpu_parity import (NAN_BITS, SENTINEL_SCORE, assert_same_contents, check_find, dev, hkv, mixed_queries,
                             np_u64, sample_present, to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def fill(tab, o, C, D, seed, stream, lam=1.0, batch=1 << 12):
    step, start = 0, 0
    target = int(round(lam * C))
    while o.size() < target:
        step += 1
        n = batch if lam >= 1.0 else min(batch, target - o.size())
        keys = gen.unique_keys(seed, stream, start, n, device=dev())
        start += n
        vals = gen.values(keys, step, D)
        sc = torch.full((n,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(keys, vals, sc)
        o.insert_or_assign(np_u64(keys), np_u64(sc), values=vals.cpu().numpy())
    return step, start


def check_find_ptr(tab, o, q, split=None):
    n = q.numel()
    ptrs = torch.full((n,), -1, dtype=torch.int64, device=dev())
    found = torch.full((n,), 7, dtype=torch.uint8, device=dev())
    scores = torch.full((n,), SENTINEL_SCORE, dtype=torch.int64, device=dev())
    tab.find_ptr(q, ptrs_out=ptrs, found_out=found, scores_out=scores)
    contains = tab.contains(q)
    torch.cuda.synchronize()
    qk = np_u64(q)
    ofound, opos = o.find_pos(qk)
    osc = np.full(n, SENTINEL_SCORE, np.uint64)
    o.find(qk, scores_out=osc)
    f = found.cpu().numpy()
    assert np.array_equal(f, ofound)
    assert np.array_equal(contains.cpu().numpy(), ofound)
    assert np.array_equal(np_u64(scores), osc)
    p = ptrs.cpu().numpy().view(np.uint64)
    assert np.all(p[f == 0] == 0)
    # every hit's address is one common base plus its slot position in rows,
    # the position being where export lists the key
    k, _, _, pos = tab.export_batch(with_values=False)
    where = dict(zip(np_u64(k).tolist(), np_u64(pos).tolist()))
    hit = np.flatnonzero(f)
    gpos = np.array([where[int(x)] for x in qk[hit]], dtype=np.uint64)
    row = np.uint64(4 * tab.dim)
    # with an HBM watermark, rows at and above `split` have a base of their own
    cut = np.uint64(tab.capacity if split is None else split)
    lo = gpos < cut
    for m, first in ((lo, np.uint64(0)), (~lo, cut)):
        base = p[hit][m] - (gpos[m] - first) * row
        assert base.size == 0 or np.all(base == base[0])
    return p, hit, gpos, opos


def test_find_ptr_and_contains_single_bucket():
    """The small single-bucket workload's table (512 buckets x 128, dim 16) at
    lambda = 1: find* and contains on half resident, half absent keys plus
    reserved keys."""
    H = hkv()
    C, D = 1 << 16, 16
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    fill(tab, o, C, D, 0x484B560000000001, 1, batch=16384)
    q = mixed_queries(o, 16384, 0.5, 3, 55)
    q = torch.cat([q, to_dev(np.array([oracle.EMPTY_KEY, oracle.LOCKED_KEY], dtype=np.uint64))])
    _, hit, _, _ = check_find_ptr(tab, o, q)
    assert hit.size == 8192


@pytest.mark.parametrize("dual", [False, True])
def test_find_ptr_serial_positions_equal_oracle(dual):
    """Serial inserts place keys in the oracle's slots, so find* addresses give
    exactly the oracle's positions; dual-bucket rows lie in a candidate bucket."""
    H = hkv()
    C, D = 16 * SLOTS, 5
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=dual)
    fill(tab, o, C, D, 9, 2, batch=700)
    q = mixed_queries(o, 3000, 0.7, 4, 56)
    p, hit, gpos, opos = check_find_ptr(tab, o, q)
    assert np.array_equal(gpos, opos[hit])
    if dual:
        b1, b2, _ = o.route(np_u64(q)[hit])
        assert np.all((gpos // SLOTS == b1) | (gpos // SLOTS == b2))


def test_find_ptr_parallel_dual_and_tiered():
    H = hkv()
    C, D = 64 * SLOTS, 8
    for host in (False, True):
        tab = H.HashTable(C, D, dual_bucket=True, values_on_host=host)
        o = oracle.OracleTable(C, D, dual=True)
        keys = gen.unique_keys(12, 1, 0, C, device=dev())
        vals = gen.values(keys, 1, D)
        sc = torch.ones(C, dtype=torch.int64, device=dev())
        tab.insert_or_assign(keys, vals, sc)
        k, _, _, pos = tab.export_batch(with_values=False)
        q = torch.cat([k[:4000], gen.unique_keys(12, 2, 0, 1000, device=dev())])
        ptrs, found = tab.find_ptr(q)
        torch.cuda.synchronize()
        f = found.cpu().numpy()
        assert f[:4000].all() and not f[4000:].any()
        p = ptrs.cpu().numpy().view(np.uint64)
        assert np.all(p[4000:] == 0)
        base = p[:4000] - np_u64(pos[:4000]) * np.uint64(4 * D)
        assert np.all(base == base[0])
        tab.close()


def evict_sets(ek, ev, es, cnt):
    torch.cuda.synchronize()
    m = int(cnt.item())
    k = np_u64(ek[:m])
    order = np.argsort(k)
    return k[order], np_u64(es[:m])[order], ev[:m].cpu().numpy()[order]


def oracle_evict_sets(out):
    order = np.argsort(out["keys"])
    return out["keys"][order], out["scores"][order], out["values"][order]


def test_insert_and_evict_single_bucket_exact():
    """lambda = 1 table (2^14 slots, dim 8). Batches of half resident, half new
    keys with rising scores (evictions), then a low-score burst (everything
    turned away, table unchanged) and a high-score burst (admitted whole)."""
    H = hkv()
    C, D = 1 << 14, 8
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    step, _ = fill(tab, o, C, D, 21, 1)
    for t in range(5):
        step += 1
        fresh = gen.unique_keys(21, 2, t * 2048, 2048).numpy().view(np.uint64)
        old = sample_present(o, 2048, 50 + t)
        k = np.random.default_rng(t).permutation(np.concatenate([fresh, old]))
        kt = to_dev(k)
        v = gen.values(kt, 100 + step, D)
        sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
        got = evict_sets(*tab.insert_and_evict(kt, v, sc))
        want = oracle_evict_sets(o.insert_and_evict(k, np_u64(sc), values=v.cpu().numpy()))
        assert want[0].size > 0
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        assert_same_contents(tab, o)
    for burst_score, stream in ((0, 3), (10 ** 6, 4)):
        k = gen.unique_keys(21, stream, 0, 1024, device=dev())
        v = gen.values(k, 7, D)
        sc = torch.full((1024,), burst_score, dtype=torch.int64, device=dev())
        got = evict_sets(*tab.insert_and_evict(k, v, sc))
        want = oracle_evict_sets(o.insert_and_evict(np_u64(k), np_u64(sc), values=v.cpu().numpy()))
        assert got[0].size == 1024
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        if burst_score == 0:
            assert np.array_equal(got[0], np.sort(np_u64(k)))
        assert_same_contents(tab, o)


def test_insert_and_evict_without_optional_outputs_and_empty():
    H = hkv()
    C, D = 8 * SLOTS, 4
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    fill(tab, o, C, D, 22, 1, batch=512)
    k = gen.unique_keys(22, 2, 0, 600, device=dev())
    v = gen.values(k, 3, D)
    sc = torch.full((600,), 99, dtype=torch.int64, device=dev())
    ek = torch.empty(600, dtype=torch.int64, device=dev())
    cnt = torch.full((1,), 12345, dtype=torch.int64, device=dev())
    hkv().hkv_insert_and_evict(tab.handle, k, v, sc, ek, None, None, cnt, dim=D, device=0)
    want = o.insert_and_evict(np_u64(k), np_u64(sc), values=v.cpu().numpy())
    torch.cuda.synchronize()
    m = int(cnt.item())
    assert np.array_equal(np.sort(np_u64(ek[:m])), np.sort(want["keys"]))
    # an empty batch only resets the count
    cnt.fill_(777)
    empty = torch.empty(0, dtype=torch.int64, device=dev())
    hkv().hkv_insert_and_evict(tab.handle, empty, torch.empty((0, D), device=dev()), empty, ek, None, None, cnt,
                               dim=D, device=0)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0
    assert_same_contents(tab, o)


@pytest.mark.parametrize("dual", [False, True])
def test_insert_and_evict_serial_same_order_and_positions(dual):
    H = hkv()
    C, D = 16 * SLOTS, 3
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=dual)
    rng = np.random.default_rng(23)
    pool = rng.integers(1, 1 << 62, size=6000, dtype=np.int64)
    for step in range(1, 12):
        k = rng.permutation(np.unique(rng.choice(pool, 700, replace=False)))
        kt = torch.from_numpy(k).to(dev())
        sc = torch.from_numpy(step * 4 + rng.integers(0, 4, size=k.size)).to(dev())
        v = gen.values(kt, step, D)
        ek, ev, es, cnt = tab.insert_and_evict(kt, v, sc)
        want = o.insert_and_evict(k.view(np.uint64), np_u64(sc), values=v.cpu().numpy())
        torch.cuda.synchronize()
        m = int(cnt.item())
        assert np.array_equal(np_u64(ek[:m]), want["keys"])
        assert np.array_equal(np_u64(es[:m]), want["scores"])
        assert np.array_equal(ev[:m].cpu().numpy().view(np.uint32), want["values"].view(np.uint32))
        gk, _, _, gp = tab.export_batch(with_values=False)
        e = o.export()
        order = np.argsort(np_u64(gp))
        assert np.array_equal(np_u64(gp)[order], e["pos"]) and np.array_equal(np_u64(gk)[order], e["keys"])
    assert_same_contents(tab, o)


def test_insert_and_evict_dual_parallel_conserves_entries():
    """Dual-bucket parallel mode under a Zipf stream with frequency scores:
    hand-back and table together hold exactly what was resident or offered,
    nothing twice, every handed-back row is that key's last written row."""
    H = hkv()
    C, D = 1 << 14, 4
    tab = H.HashTable(C, D, dual_bucket=True)
    z = gen.Zipf(1.05, 1 << 18)
    freq = {}
    resident = set()
    for b in range(16):
        r = z.draw(78, 1, b * 4096, 4096).numpy()
        uniq, cnt_ = np.unique(r, return_counts=True)
        for x, c in zip(uniq.tolist(), cnt_.tolist()):
            freq[x] = freq.get(x, 0) + c
        keys = uniq.astype(np.uint64)
        sc = np.array([freq[x] for x in uniq.tolist()], dtype=np.uint64)
        kt, st = to_dev(keys), to_dev(sc)
        v = gen.values(kt, st, D)
        ek, ev, es, cnt = tab.insert_and_evict(kt, v, st)
        torch.cuda.synchronize()
        m = int(cnt.item())
        out = np_u64(ek[:m])
        gk, _, _, _ = tab.export_batch(with_values=False)
        after = set(np_u64(gk).tolist())
        assert np.unique(out).size == m
        assert not (set(out.tolist()) & after)
        assert set(out.tolist()) | after == resident | set(keys.tolist())
        assert m <= len(set(keys.tolist()) - resident)
        assert all(freq[x] == s for x, s in zip(out.tolist(), np_u64(es[:m]).tolist()))
        assert torch.equal(ev[:m], gen.values(ek[:m], es[:m], D))
        resident = after


def test_find_or_insert_single_bucket_exact():
    """lambda = 1 table (2^14 slots, dim 8): batches of half resident, half new
    keys; found flags, returned rows (stored rows of hits, untouched rows of
    misses) and table contents exact."""
    H = hkv()
    C, D = 1 << 14, 8
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    step, _ = fill(tab, o, C, D, 24, 1)
    for t in range(5):
        step += 1
        fresh = gen.unique_keys(24, 2, t * 2048, 2048).numpy().view(np.uint64)
        old = sample_present(o, 2048, 60 + t)
        k = np.random.default_rng(t).permutation(np.concatenate([fresh, old]))
        kt = to_dev(k)
        v = gen.values(kt, 100 + step, D)
        v0 = v.cpu().numpy()
        sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
        rows, found = tab.find_or_insert(kt, v, sc)
        orows, ofound = o.find_or_insert(k, np_u64(sc), values=v0)
        torch.cuda.synchronize()
        assert np.array_equal(found.cpu().numpy(), ofound)
        assert ofound.sum() == 2048
        assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        assert_same_contents(tab, o)


@pytest.mark.parametrize("dual", [False, True])
def test_find_or_insert_serial_positions(dual):
    H = hkv()
    C, D = 16 * SLOTS, 4
    tab = H.HashTable(C, D, dual_bucket=dual, serial_insert=True)
    o = oracle.OracleTable(C, D, dual=dual)
    rng = np.random.default_rng(25)
    pool = rng.integers(1, 1 << 62, size=5000, dtype=np.int64)
    for step in range(1, 10):
        k = rng.permutation(np.unique(rng.choice(pool, 600, replace=False)))
        kt = torch.from_numpy(k).to(dev())
        sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
        v = gen.values(kt, step, D)
        v0 = v.cpu().numpy()
        rows, found = tab.find_or_insert(kt, v, sc)
        orows, ofound = o.find_or_insert(k.view(np.uint64), np_u64(sc), values=v0)
        torch.cuda.synchronize()
        assert np.array_equal(found.cpu().numpy(), ofound)
        assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        gk, _, _, gp = tab.export_batch(with_values=False)
        e = o.export()
        order = np.argsort(np_u64(gp))
        assert np.array_equal(np_u64(gp)[order], e["pos"]) and np.array_equal(np_u64(gk)[order], e["keys"])
    assert_same_contents(tab, o)


def test_find_or_insert_odd_dim_and_reserved_keys():
    H = hkv()
    C, D = 8 * SLOTS, 3
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    fill(tab, o, C, D, 26, 1, batch=500)
    k = np.concatenate([sample_present(o, 300, 1), gen.unique_keys(26, 2, 0, 300).numpy().view(np.uint64),
                        np.array([oracle.EMPTY_KEY, oracle.LOCKED_KEY], dtype=np.uint64)])
    kt = to_dev(k)
    v = gen.values(kt, 50, D)
    v0 = v.cpu().numpy()
    sc = torch.full((k.size,), 50, dtype=torch.int64, device=dev())
    rows, found = tab.find_or_insert(kt, v, sc)
    orows, ofound = o.find_or_insert(k, np_u64(sc), values=v0)
    torch.cuda.synchronize()
    assert np.array_equal(found.cpu().numpy(), ofound)
    assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
    assert_same_contents(tab, o)


# ------------------------------------------------ HBM watermark value split --

def _memory_type(addr):
    """hipPointerGetAttributes(...).type of a device-visible address: 1 host, 2 device."""
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    buf = (ctypes.c_int32 * 16)()
    assert hip.hipPointerGetAttributes(buf, ctypes.c_void_p(int(addr))) == 0
    return int(buf[0])


@pytest.mark.parametrize("dual", [False, True])
def test_hbm_watermark_split_exact(dual):
    """values_on_host with an HBM budget of 20 buckets' rows (plus change):
    the first 20 buckets' rows are in HBM, the rest in pinned host memory.
    Contents, find and find* must match the oracle exactly (single mode; dual
    mode serial), and find* addresses must lie in device memory below the
    split and in host memory above it."""
    H = hkv()
    B, D = 64, 8
    C = B * SLOTS
    budget = 20 * SLOTS * 4 * D + 100
    split = 20 * SLOTS
    tab = H.HashTable(C, D, dual_bucket=dual, values_on_host=True, hbm_value_bytes=budget, serial_insert=dual)
    o = oracle.OracleTable(C, D, dual=dual)
    fill(tab, o, C, D, 27, 1, batch=1500)
    assert_same_contents(tab, o)
    q = mixed_queries(o, 4000, 0.8, 7, 57)
    from test_gpu_parity import check_find

    check_find(tab, o, q)
    p, hit, gpos, _ = check_find_ptr(tab, o, q, split=split)
    lo, hi = hit[gpos < split], hit[gpos >= split]
    assert lo.size > 100 and hi.size > 100
    row = np.uint64(4 * D)
    base_lo = p[lo] - gpos[gpos < split] * row
    base_hi = p[hi] - (gpos[gpos >= split] - np.uint64(split)) * row
    assert np.all(base_lo == base_lo[0]) and np.all(base_hi == base_hi[0])
    assert _memory_type(p[lo][0]) == 2 and _memory_type(p[hi][0]) == 1
    # updates and an eviction-heavy round go through the split too
    k = gen.unique_keys(27, 9, 0, 2000, device=dev())
    v = gen.values(k, 99, D)
    sc = torch.full((2000,), 10 ** 6, dtype=torch.int64, device=dev())
    got = evict_sets(*tab.insert_and_evict(k, v, sc))
    want = oracle_evict_sets(o.insert_and_evict(np_u64(k), np_u64(sc), values=v.cpu().numpy()))
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    assert_same_contents(tab, o)


def test_hbm_watermark_extremes():
    """Budget 0 keeps every row on the host, a budget of the whole table keeps
    every row in HBM, values_on_host = 0 ignores the budget."""
    H = hkv()
    C, D = 8 * SLOTS, 4
    for host, budget, want in ((True, 0, 1), (True, C * 4 * D, 2), (False, 123, 2)):
        tab = H.HashTable(C, D, values_on_host=host, hbm_value_bytes=budget)
        o = oracle.OracleTable(C, D)
        fill(tab, o, C, D, 28, 1, batch=512)
        assert_same_contents(tab, o)
        k, _, _, _ = tab.export_batch(with_values=False)
        ptrs, found = tab.find_ptr(k[:64])
        torch.cuda.synchronize()
        assert found.all()
        assert {_memory_type(x) for x in ptrs.cpu().numpy().view(np.uint64).tolist()} == {want}
        tab.close()


# --------------------------------- concurrent reader/updater/inserter threads --

@pytest.mark.parametrize("rw_lock", [False, True])
def test_mixed_threads_keep_the_table_consistent(rw_lock):
    """The native multi-threaded driver: 3 finders, 3 updaters and 2 inserters
    on streams of their own, 30 batches each, on one table ordered by the
    three groups (or the reader/writer baseline). Afterwards: no key twice,
    at most 128 per bucket, every key in its own bucket, every row the
    generated row of a version written for that key, every score one that
    was written."""
    import ctypes

    from hash_table_cache_amd import build as hb

    H = hkv()
    C, D, batch, pool, nb = 64 * SLOTS, 8, 1024, 3, 30
    tab = H.HashTable(C, D, flags=H.HKV_FLAG_RW_LOCK if rw_lock else 0)
    o = oracle.OracleTable(C, D)
    fill(tab, o, C, D, 29, 1, lam=0.75, batch=2048)
    k_all, _, _, _ = tab.export_batch(with_values=False)
    roles = "FFFUUUII"
    bufs, ptrs = [], {n: [] for n in ("keys", "values", "scores", "out", "found")}
    for j, r in enumerate(roles):
        pick = torch.argsort(gen.counter_words(29, 40 + j, 0, k_all.numel(), dev()))[:pool * batch]
        k = k_all[pick]
        if r == "I":
            fresh = gen.unique_keys(29, 60 + j, 0, pool * batch // 2, device=dev())
            k = torch.cat([k[:pool * batch // 2], fresh]).contiguous()
        ver = torch.full((pool * batch,), 1000 + j, dtype=torch.int64, device=dev())
        v = gen.values(k, ver, D)
        sc = torch.full((pool * batch,), 10 ** 6, dtype=torch.int64, device=dev())
        o_, f_ = torch.empty((batch, D), device=dev()), torch.empty(batch, dtype=torch.uint8, device=dev())
        bufs.append((k, v, sc, o_, f_))
        for n, t in zip(("keys", "values", "scores", "out", "found"), (k, v, sc, o_, f_)):
            ptrs[n].append(t.data_ptr())
    torch.cuda.synchronize()
    lib = ctypes.CDLL(str(hb.MIXED_LIB_PATH))
    P = ctypes.c_void_p
    lib.hkv_mixed_run.argtypes = [P, ctypes.c_uint32, P, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32,
                                  P, P, P, P, P, ctypes.POINTER(ctypes.c_double)]
    arr = {n: (ctypes.c_void_p * len(roles))(*v) for n, v in ptrs.items()}
    role_ids = (ctypes.c_int32 * len(roles))(*["FUI".index(r) for r in roles])
    secs = ctypes.c_double(0)
    st = lib.hkv_mixed_run(tab.handle, len(roles), role_ids, nb, batch, pool, arr["keys"], arr["values"],
                           arr["scores"], arr["out"], arr["found"], ctypes.byref(secs))
    assert st == 0 and secs.value > 0
    gk, gv, gs, gp = tab.export_batch()
    ku, pu = np_u64(gk), np_u64(gp)
    assert np.unique(ku).size == ku.size and tab.size() == ku.size <= C
    assert np.bincount((pu // SLOTS).astype(np.int64)).max() <= SLOTS
    b1 = o.route(ku)[0]
    assert np.array_equal(pu // SLOTS, b1)
    # versions written: 1 (fill) or 1000 + j of the updater / inserter threads
    kt = gk
    ok = torch.zeros(ku.size, dtype=torch.bool, device=dev())
    for ver in [None] + [1000 + j for j, r in enumerate(roles) if r != "F"]:
        if ver is None:
            cand = torch.stack([gen.values(kt, s, D) for s in range(1, 5)])  # fill steps
            ok |= (cand == gv.unsqueeze(0)).all(-1).any(0)
        else:
            ok |= (gen.values(kt, torch.full_like(kt, ver), D) == gv).all(-1)
    assert bool(ok.all())
    # scores: the fill's step or the threads' 10^6
    s_ = np_u64(gs)
    assert np.all((s_ == 10 ** 6) | (s_ <= 4))


@pytest.mark.parametrize("budget_buckets", [0, 8])
def test_host_rows_read_again_after_updates(budget_buckets):
    """Rows on the host are read with cacheable loads. Hot keys are found many
    times in one batch, then rewritten by assign, insert_or_assign and
    find_or_insert between finds; every find must return the newest rows."""
    H = hkv()
    C, D = 32 * SLOTS, 16
    tab = H.HashTable(C, D, values_on_host=True, hbm_value_bytes=budget_buckets * SLOTS * 4 * D)
    o = oracle.OracleTable(C, D)
    fill(tab, o, C, D, 31, 1, batch=1024)
    from test_gpu_parity import check_find

    hot = sample_present(o, 64, 3)
    q = to_dev(np.repeat(hot, 64))  # every hot key 64 times in one batch
    for r in range(4):
        check_find(tab, o, q)
        v = gen.values(to_dev(hot), 500 + r, D)
        sc = torch.full((hot.size,), 100 + r, dtype=torch.int64, device=dev())
        if r % 3 == 0:
            tab.assign(to_dev(hot), v, sc)
            o.assign(hot, values=v.cpu().numpy(), scores=np_u64(sc))
        elif r % 3 == 1:
            tab.insert_or_assign(to_dev(hot), v, sc)
            o.insert_or_assign(hot, np_u64(sc), values=v.cpu().numpy())
        else:
            rows, _ = tab.find_or_insert(to_dev(hot), v.clone(), sc)
            orows, _ = o.find_or_insert(hot, np_u64(sc), values=v.cpu().numpy())
            torch.cuda.synchronize()
            assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
    check_find(tab, o, q)
    assert_same_contents(tab, o)


@pytest.mark.parametrize("D,dual", [(5, False), (33, False), (64, True)])
def test_host_rows_find_partitioned_over_xcds(D, dual):
    """With rows in host memory, find serves each chunk of keys with one
    workgroup per XCD, each taking the keys of its hash class. Ragged batch
    sizes, repeated keys, odd dims (scalar row copies) and dual mode must give
    the oracle's flags, rows and scores exactly."""
    H = hkv()
    C = 24 * SLOTS
    tab = H.HashTable(C, D, dual_bucket=dual, values_on_host=True, serial_insert=dual)
    o = oracle.OracleTable(C, D, dual=dual)
    fill(tab, o, C, D, 41, 1, batch=1100)
    from test_gpu_parity import check_find

    for n, seed in ((1, 3), (257, 4), (3001, 5)):
        q = mixed_queries(o, n, 0.7, seed, 60 + seed)
        check_find(tab, o, q)
    hot = sample_present(o, 16, 8)
    check_find(tab, o, to_dev(np.repeat(hot, 40)))


@pytest.mark.parametrize("D", [1, 5, 33])
def test_insert_and_evict_and_find_or_insert_odd_dims(D):
    """Rows that are not a whole number of 16-byte pieces take the scalar copy
    paths of the staging, compaction and fetch kernels."""
    H = hkv()
    C = 16 * SLOTS
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    step, _ = fill(tab, o, C, D, 32, 1, batch=1000)
    for t in range(3):
        step += 1
        fresh = gen.unique_keys(32, 2 + t, 0, 700).numpy().view(np.uint64)
        k = np.random.default_rng(t).permutation(np.concatenate([fresh, sample_present(o, 500, 70 + t)]))
        kt = to_dev(k)
        v = gen.values(kt, 300 + step, D)
        sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
        if t % 2 == 0:
            got = evict_sets(*tab.insert_and_evict(kt, v, sc))
            want = oracle_evict_sets(o.insert_and_evict(k, np_u64(sc), values=v.cpu().numpy()))
            assert got[0].size > 0 and np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
            assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        else:
            v0 = v.cpu().numpy()
            rows, found = tab.find_or_insert(kt, v, sc)
            orows, ofound = o.find_or_insert(k, np_u64(sc), values=v0)
            torch.cuda.synchronize()
            assert np.array_equal(found.cpu().numpy(), ofound)
            assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        assert_same_contents(tab, o)


@pytest.mark.parametrize("D", [129, 132, 256, 260])
def test_wide_rows_every_call_exact(D):
    """Rows wider than 128 floats: the row copies loop over several 512-byte
    pieces per 16 lanes, and the inserter's owner copies rows from the input
    instead of holding them in registers, on every path (update, empty slot,
    eviction, rejection, staging of evicted rows). 129 takes the scalar copy."""
    H = hkv()
    C = 16 * SLOTS
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    step, _ = fill(tab, o, C, D, 41, 1, batch=1000)
    assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 700, 0.7, 5, 11))
    step += 1
    absent = gen.unique_keys(41, 9, 0, 100).numpy().view(np.uint64)
    ak = np.random.default_rng(1).permutation(np.concatenate([sample_present(o, 400, 3), absent]))
    akt = to_dev(ak)
    av = gen.values(akt, 500 + step, D)
    asc = torch.full((ak.size,), step, dtype=torch.int64, device=dev())
    tab.assign(akt, av, asc)
    o.assign(ak, values=av.cpu().numpy(), scores=np_u64(asc))
    assert_same_contents(tab, o)
    for t in range(4):
        step += 1
        fresh = gen.unique_keys(41, 20 + t, 0, 600).numpy().view(np.uint64)
        k = np.random.default_rng(10 + t).permutation(np.concatenate([fresh, sample_present(o, 600, 80 + t)]))
        kt = to_dev(k)
        v = gen.values(kt, 600 + step, D)
        # odd calls offer scores below every resident's, so admission turns
        # the new keys away
        sc = torch.full((k.size,), step if t % 2 == 0 else 0, dtype=torch.int64, device=dev())
        if t < 2:
            got = evict_sets(*tab.insert_and_evict(kt, v, sc))
            want = oracle_evict_sets(o.insert_and_evict(k, np_u64(sc), values=v.cpu().numpy()))
            assert got[0].size > 0 and np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
            assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        else:
            v0 = v.cpu().numpy()
            rows, found = tab.find_or_insert(kt, v, sc)
            orows, ofound = o.find_or_insert(k, np_u64(sc), values=v0)
            torch.cuda.synchronize()
            assert np.array_equal(found.cpu().numpy(), ofound)
            assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
        assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 700, 0.7, 6, 12))


def test_largest_row_width_every_call_exact():
    """Rows of the largest width a table accepts (2^20 floats, 4 MiB each) in
    one bucket: inserts that fill it and then evict, find with scores,
    insert_and_evict, find_or_insert and assign, every result and the table's
    contents bit-exact against the oracle (64-bit row offsets, long row-copy
    loops, long chains of one owner)."""
    H = hkv()
    C, D = SLOTS, 1 << 20
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    step = 0
    for b in range(3):  # 144 distinct keys into 128 slots
        step += 1
        k = gen.unique_keys(47, 1, 48 * b, 48, device=dev())
        v = gen.values(k, step, D)
        sc = torch.full((48,), step, dtype=torch.int64, device=dev())
        tab.insert_or_assign(k, v, sc)
        o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
        del v
    assert o.size() == C
    assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 24, 0.75, 5, 47))
    step += 1
    k = gen.unique_keys(47, 2, 0, 16, device=dev())
    v = gen.values(k, step, D)
    sc = torch.full((16,), step, dtype=torch.int64, device=dev())
    got = evict_sets(*tab.insert_and_evict(k, v, sc))
    want = oracle_evict_sets(o.insert_and_evict(np_u64(k), np_u64(sc), values=v.cpu().numpy()))
    assert got[0].size == 16 and np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    del got, want, v
    step += 1
    fresh = gen.unique_keys(47, 3, 0, 8).numpy().view(np.uint64)
    k = np.random.default_rng(47).permutation(np.concatenate([fresh, sample_present(o, 8, 48)]))
    kt = to_dev(k)
    v = gen.values(kt, step, D)
    sc = torch.full((k.size,), step, dtype=torch.int64, device=dev())
    v0 = v.cpu().numpy()
    rows, found = tab.find_or_insert(kt, v, sc)
    orows, ofound = o.find_or_insert(k, np_u64(sc), values=v0)
    torch.cuda.synchronize()
    assert np.array_equal(found.cpu().numpy(), ofound)
    assert np.array_equal(rows.cpu().numpy().view(np.uint32), orows.view(np.uint32))
    del rows, orows, v, v0
    step += 1
    ak = sample_present(o, 16, 49)
    akt = to_dev(ak)
    av = gen.values(akt, step, D)
    asc = torch.full((ak.size,), step, dtype=torch.int64, device=dev())
    tab.assign(akt, av, asc)
    o.assign(ak, values=av.cpu().numpy(), scores=np_u64(asc))
    del av
    assert_same_contents(tab, o)
    check_find(tab, o, mixed_queries(o, 24, 0.75, 6, 50))
    tab.close()


def test_find_or_insert_dual_parallel_invariants():
    """Dual-bucket parallel find_or_insert under a Zipf stream: found iff the
    key was resident before, hits return the row of the key's last write,
    and the table keeps its invariants (no key twice, every entry in a
    candidate bucket, rows and scores of the last write)."""
    H = hkv()
    C, D = 1 << 13, 4
    tab = H.HashTable(C, D, dual_bucket=True)
    o = oracle.OracleTable(C, D, dual=True)
    z = gen.Zipf(1.1, 1 << 16)
    last = {}
    for b in range(12):
        keys = np.unique(z.draw(79, 1, b * 2048, 2048).numpy()).astype(np.uint64)
        kt = to_dev(keys)
        sc = torch.full((keys.size,), b + 1, dtype=torch.int64, device=dev())
        rows = gen.values(kt, sc, D)
        offered = rows.clone()
        gk, _, _, _ = tab.export_batch(with_values=False)
        before = set(np_u64(gk).tolist())
        rows, found = tab.find_or_insert(kt, rows, sc)
        torch.cuda.synchronize()
        f = found.cpu().numpy().astype(bool)
        assert np.array_equal(f, np.array([x in before for x in keys.tolist()]))
        hv = torch.tensor([last[x] for x in keys[f].tolist()], dtype=torch.int64)
        assert torch.equal(rows[torch.from_numpy(f).to(dev())].cpu(), gen.values(kt[torch.from_numpy(f).to(dev())].cpu(), hv, D))
        assert torch.equal(rows[torch.from_numpy(~f).to(dev())], offered[torch.from_numpy(~f).to(dev())])
        for x, hit in zip(keys.tolist(), f.tolist()):
            if not hit:
                last[x] = b + 1  # inserted rows are version b + 1; hits keep their row version
        gk, gv, gs, gp = tab.export_batch()
        ku, pu = np_u64(gk), np_u64(gp)
        assert np.unique(ku).size == ku.size and tab.size() == ku.size <= C
        b1, b2, _ = o.route(ku)
        assert np.all((pu // SLOTS == b1) | (pu // SLOTS == b2))
        ver = torch.tensor([last[x] for x in ku.tolist()], dtype=torch.int64, device=dev())
        assert torch.equal(gv, gen.values(gk, ver, D))
        assert np.all(np_u64(gs) >= 1)
