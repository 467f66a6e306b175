"""Full-size GPU checks, in the launch configuration the benchmark uses.

At these sizes the oracle cannot replay whole workloads in test time, so the
checks are (a) exact against the closed form of single-bucket mode (distinct
keys per batch, scores never decreasing): every bucket holds exactly the top
128 by (score, key) of every key routed there, compared on all buckets with
library sorts (tests/closed_form.py), and exact on every find output (found
iff resident by the closed form, row = the row generated for the key's last
write, score = last written score), and (b) invariants at any size: no key
resident twice, at most 128 entries per bucket, every entry in one of its
candidate buckets, size = exported count <= capacity, and for dual-bucket
mode top-N retention against the ideal top N by (score, key).

Bucket routing of the expected sets comes from the oracle's route function.
The inputs of every step (resident keys to query, update or re-insert) are
drawn from the closed form's resident set, not from the table.
"""

import time

import numpy as np
import pytest
import torch

import closed_form as cf
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


def u64(t):
    return t.detach().cpu().numpy().view(np.uint64)


def log(msg):
    print(f"[full-size] {msg}", flush=True)


def route_all(keys_np, capacity, dual=False):
    """(b1, b2) of keys under a table of `capacity` slots (oracle routing)."""
    b1, b2, _ = oracle.route_buckets(keys_np, capacity // SLOTS, dual)
    return b1, b2


def export_all(tab, with_values=False):
    k, v, s, p = tab.export_batch(with_values=with_values)
    return k, v, s, p


def check_invariants(tab, k, p, capacity):
    n = k.numel()
    assert tab.size() == n <= capacity
    assert torch.unique(k).numel() == n, "a key is resident twice"
    counts = torch.bincount(torch.div(p, SLOTS, rounding_mode="floor"), minlength=capacity // SLOTS)
    assert int(counts.max()) <= SLOTS


def check_find_exact(tab, q, resident_sorted, version_of):
    """find outputs against the exported table: found iff resident, row = the
    generated row of (key, version), score = version, misses untouched."""
    n = q.numel()
    d = tab.dim
    nan = torch.full((n, d), 0x7FC00BAD, dtype=torch.int32, device=dev()).view(torch.float32)
    sent = torch.full((n,), 0x5EED, dtype=torch.int64, device=dev())
    vals, found, scores = tab.find(q, values_out=nan, scores_out=sent)
    torch.cuda.synchronize()
    idx = torch.searchsorted(resident_sorted, q)
    idx = torch.clamp(idx, max=resident_sorted.numel() - 1)
    expect = resident_sorted[idx] == q
    assert torch.equal(found.bool(), expect)
    f = expect
    ver = version_of(q[f])
    assert torch.equal(scores[f], ver)
    assert torch.equal(vals[f].view(torch.int32), gen.values(q[f], ver, d).view(torch.int32))
    assert bool((vals[~f].view(torch.int32) == 0x7FC00BAD).all())
    assert bool((scores[~f] == 0x5EED).all())
    return int(f.sum())


@pytest.mark.parametrize("lam,cap_log2,D", [(0.5, 26, 64), (1.0, 26, 64), (1.0, 28, 64), (0.75, 26, 32),
                                             (0.9, 26, 32)])
def test_lambda_sweep_table_at_full_size(lam, cap_log2, D):
    """2^26 slots (and 2^28, the largest capacity of the workloads, with its
    64 GiB of rows in HBM), dim 64 and the λ-sweep workload's own dim 32,
    single bucket: fill with distinct uniform keys in 2^20 batches (score =
    batch index; the size after every batch equal to the closed form's),
    then the exact contents of every bucket, an exact 2^20-key find (90 %
    resident), one upsert step (90 % resident, 10 % new), and the checks
    again."""
    H = hkv()
    cap, batch = 1 << cap_log2, 1 << 20
    seed = 0x484B56000000AA00 + int(lam * 100) + cap_log2
    tab = H.HashTable(cap, D)
    t0 = time.time()
    target = int(lam * cap)
    cursor, step = 0, 0
    score_parts = []
    fill = cf.FillCount(cap, dev())
    while fill.size() < target:
        n = batch if lam >= 1.0 else min(batch, target - fill.size())
        step += 1
        k = gen.unique_keys(seed, 1, cursor, n, device=dev())
        tab.insert_or_assign(k, gen.values(k, step, D), torch.full((n,), step, dtype=torch.int64, device=dev()))
        score_parts.append((cursor, n, step))
        cursor += n
        assert tab.size() == fill.add(k), f"size after batch {step} differs from the closed form"
    log(f"lambda {lam}, 2^{cap_log2} slots: {cursor} keys in {step} batches, size {tab.size()}, "
        f"{time.time() - t0:.1f}s")
    allk = gen.unique_keys(seed, 1, 0, cursor, device=dev())
    alls = torch.cat([torch.full((n,), st, dtype=torch.int64, device=dev()) for _, n, st in score_parts])

    def check(allk, alls):
        k, _, s, p = export_all(tab)
        check_invariants(tab, k, p, cap)
        # every resident key's score is its last written score
        order = torch.argsort(allk)
        sk, ss = allk[order], alls[order]
        pos = torch.searchsorted(sk, k)
        assert torch.equal(sk[pos], k)
        assert torch.equal(ss[pos], s)
        # every bucket: exactly the top 128 by (score, key) of the keys routed there
        resident = cf.assert_table_matches(k, p, allk, alls, cap)
        log(f"lambda {lam}, 2^{cap_log2} slots: all {cap // SLOTS} buckets equal the closed form "
            f"({resident.numel()} entries)")
        return resident

    resident = check(allk, alls)
    # exact find, 90 % resident (recent keys), 10 % never inserted
    rng = torch.Generator(device="cpu").manual_seed(5)
    hits = resident[torch.randperm(resident.numel(), generator=rng)[: int(0.9 * batch)].to(dev())]
    miss = gen.unique_keys(seed, 7, 0, batch - hits.numel(), device=dev())
    q = gen.shuffle(torch.cat([hits, miss]), seed, 8)
    order = torch.argsort(allk)
    sk, ss = allk[order], alls[order]

    def version(keys):
        return ss[torch.searchsorted(sk, keys)]

    nf = check_find_exact(tab, q, resident, version)
    assert nf == hits.numel()
    # one upsert step: 90 % resident keys re-written, 10 % new
    step += 1
    res = resident[torch.randperm(resident.numel(), generator=rng)[: int(0.9 * batch)].to(dev())]
    new = gen.unique_keys(seed, 1, cursor, batch - res.numel(), device=dev())
    uk = gen.shuffle(torch.cat([res, new]), seed, 9)
    tab.count_outcomes()
    tab.insert_or_assign(uk, gen.values(uk, step, D), torch.full((batch,), step, dtype=torch.int64, device=dev()))
    allk2 = torch.cat([allk, new])
    alls2 = torch.cat([alls, torch.full((new.numel(),), step, dtype=torch.int64, device=dev())])
    # re-written keys carry the new score
    o2 = torch.argsort(allk2)
    sk2, ss2 = allk2[o2], alls2[o2].clone()
    ss2[torch.searchsorted(sk2, res)] = step
    resident2 = check(sk2, ss2)
    # the step's outcome counts, from the closed form's states before and after
    want = {"updated": res.numel(), "inserted": int((~torch.isin(resident2, resident)).sum()),
            "evicted": int((~torch.isin(resident, resident2)).sum()),
            "rejected": int((~torch.isin(new, resident2)).sum())}
    assert tab.outcomes() == want
    log(f"lambda {lam}, 2^{cap_log2} slots: upsert step outcomes {want}")
    tab.close()


def test_continuous_online_dual_bucket_zipf_retention():
    """2^27 slots, dim 64, dual bucket; keys drawn Zipf(1.05) over 2^30 ids,
    2^20 draws per batch deduplicated, score = cumulative frequency (LFU),
    value version = score. Warm up until size == capacity, then 200 batches.
    Invariants after the run, exact find on a sampled batch, and top-N
    retention >= 0.99 against the ideal top N by (frequency, key)."""
    H = hkv()
    cap, D, draws, n_ids = 1 << 27, 64, 1 << 20, 1 << 30
    seed = 0x484B560000000003
    tab = H.HashTable(cap, D, dual_bucket=True)
    zipf = gen.Zipf(1.05, n_ids)
    freq = torch.zeros(n_ids + 1, dtype=torch.int64, device=dev())
    t0 = time.time()
    b = 0
    first_evict = None
    steady = 0
    ins_ms = 0.0
    ins_keys = 0
    size = 0
    kernels = None
    while steady < 200:
        if size >= cap and kernels is None:
            kernels = {}
            tab.profile_start()
        r = zipf.draw(seed, 1, b * draws, draws, device=dev())
        uniq, cnt = torch.unique(r, return_counts=True)
        fresh = int((freq[uniq] == 0).sum())
        freq.index_add_(0, uniq, cnt)
        sc = freq[uniq]
        v = gen.values(uniq, sc, D)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tab.insert_or_assign(uniq, v, sc)
        e1.record()
        new_size = tab.size()
        if first_evict is None and new_size - size < fresh:
            first_evict = size / cap
        if size >= cap:
            steady += 1
            ins_ms += e0.elapsed_time(e1)
            ins_keys += uniq.numel()
        size = new_size
        assert size <= cap
        b += 1
        if b > 2000:
            raise AssertionError("table never reached full capacity")
    kernels = tab.profile_stop()
    log("dual zipf: steady-state kernels " + ", ".join(f"{n} {v[1] / v[0]:.3f} ms" for n, v in kernels.items()))
    log(f"dual zipf: {b} batches ({b - 200} to fill), first eviction at lambda {first_evict:.4f}, "
        f"{time.time() - t0:.1f}s; steady-state insert_or_assign {ins_keys / ins_ms / 1e6:.3f} B-KV/s "
        f"({ins_keys / 200:.0f} distinct keys per batch)")
    k, v, s, p = export_all(tab)
    check_invariants(tab, k, p, cap)
    assert torch.equal(s, freq[k])
    # every entry sits in one of its two candidate buckets
    kn = u64(k)
    b1, b2 = route_all(kn, cap, dual=True)
    bk = u64(p) // SLOTS
    assert np.all((bk == b1) | (bk == b2))
    # sampled rows are the rows generated for (key, frequency)
    pick = torch.randperm(k.numel(), device=dev())[:200000]
    vs = torch.empty((pick.numel(), D), dtype=torch.float32, device=dev())
    vals, found, scs = tab.find(k[pick], values_out=vs, with_scores=True)
    assert bool(found.bool().all())
    assert torch.equal(vals.view(torch.int32), gen.values(k[pick], freq[k[pick]], D).view(torch.int32))
    # top-N retention: ideal = the cap highest (frequency, key) among all keys seen
    seen = torch.nonzero(freq > 0).flatten()
    fs = freq[seen]
    # rank by frequency, ties by the larger key: sort by key ascending then stable by frequency
    o = torch.argsort(seen, descending=True)
    o = o[torch.argsort(fs[o], descending=True, stable=True)]
    ideal = seen[o[:cap]]
    mark = torch.zeros(n_ids + 1, dtype=torch.bool, device=dev())
    mark[ideal] = True
    retained = int(mark[k].sum())
    retention = retained / cap
    log(f"dual zipf: top-N retention {retention:.5f} (N = {cap}, {seen.numel()} distinct keys seen)")
    assert retention >= 0.99
    # exact find on a batch of drawn keys (resident or not)
    q = torch.unique(zipf.draw(seed, 2, 0, draws, device=dev()))
    check_find_exact(tab, q, torch.sort(k).values, lambda kk: freq[kk])
    tab.close()


def test_tiered_values_dual_bucket_zipf():
    """Values in pinned, GPU-mapped host memory, dual bucket, dim 128, keys
    Zipf(1.2) over 2^32 ids, LRU scores (value version = score). Capacity 2^27
    as in the benchmark (64 GiB of pinned rows; the workload's 2^28 needs
    128 GiB, more than the host pins). Warm cache: ranks 1 .. 1.0625 *
    capacity in 2^19 batches from the coldest down to the hottest, so that
    with LRU scores the hottest ranks are the most recent; then 5 + 20 steps
    of a 2^20-draw find and a 2^19-draw upsert, the benchmark's step count.
    Invariants, and an exact find every step against the exported table."""
    H = hkv()
    cap, D = 1 << 27, 128
    seed = 0x484B560000000005
    tab = H.HashTable(cap, D, dual_bucket=True, values_on_host=True)
    t0 = time.time()
    step = 0
    hi = cap + cap // 16
    while hi > 0:
        step += 1
        lo = max(1, hi - (1 << 19) + 1)
        k = torch.arange(hi, lo - 1, -1, dtype=torch.int64, device=dev())
        hi = lo - 1
        tab.insert_or_assign(k, gen.values(k, step, D), torch.full((k.numel(),), step, dtype=torch.int64, device=dev()))
    log(f"tiered: filled ranks {cap + cap // 16}..1 in {step} batches, size {tab.size()}, {time.time() - t0:.1f}s")
    zipf = gen.Zipf(1.2, 1 << 32)
    f_ms, f_keys = 0.0, 0
    warm, steps = 5, 20
    for j in range(warm + steps):
        step += 1
        q = zipf.draw(seed, 1, j * (1 << 20), 1 << 20, device=dev())
        k, _, s, p = export_all(tab)
        resident = torch.sort(k).values
        ks, ss = torch.sort(k)
        sc_sorted = s[ss]

        def version(keys):
            return sc_sorted[torch.searchsorted(resident, keys)]

        out = torch.empty((q.numel(), D), dtype=torch.float32, device=dev())
        fnd = torch.empty(q.numel(), dtype=torch.uint8, device=dev())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tab.find(q, values_out=out, found_out=fnd)
        e1.record()
        torch.cuda.synchronize()
        if j >= warm:
            f_ms += e0.elapsed_time(e1)
            f_keys += q.numel()
        hits = check_find_exact(tab, q, resident, version)
        if j % 5 == 4:
            log(f"tiered: step {j}: {hits}/{q.numel()} hits, size {k.numel()}")
        u = torch.unique(zipf.draw(seed, 2, j * (1 << 19), 1 << 19, device=dev()))
        tab.insert_or_assign(u, gen.values(u, step, D), torch.full((u.numel(),), step, dtype=torch.int64, device=dev()))
    k, _, s, p = export_all(tab)
    check_invariants(tab, k, p, cap)
    b1, b2 = route_all(u64(k), cap, dual=True)
    bk = u64(p) // SLOTS
    assert np.all((bk == b1) | (bk == b2))
    log(f"tiered: find {f_keys / f_ms / 1e6:.4f} B-KV/s ({f_ms / steps:.2f} ms per 2^20-key batch, "
        f"rows over the host link)")
    tab.close()


def test_mixed_reader_updater_inserter_at_full_size():
    """2^27 slots, dim 64, single bucket, lambda = 1: fill with distinct
    uniform keys (score = step; size after every batch = the closed form's),
    then 5 + 20 steps, each in this order: a find of 2^20 keys (90 %
    resident), an assign of 2^19 resident keys (new row, score = step), an
    insert_or_assign of 2^18 keys (half new, half resident, score = step).
    Resident keys are drawn from the closed form's resident set. Exact find
    after every step (found iff resident by the closed form, rows of the last
    writes); at the end every bucket equals the closed form and every score
    is the last written one. Throughput of each call is logged."""
    H = hkv()
    cap, D = 1 << 27, 64
    seed = 0x484B560000000004
    tab = H.HashTable(cap, D)
    step, cursor = 0, 0
    fill = cf.FillCount(cap, dev())
    while fill.size() < cap:
        step += 1
        k = gen.unique_keys(seed, 1, cursor, 1 << 20, device=dev())
        cursor += 1 << 20
        tab.insert_or_assign(k, gen.values(k, step, D), torch.full((k.numel(),), step, dtype=torch.int64, device=dev()))
        assert tab.size() == fill.add(k)
    log(f"mixed: filled with {cursor} keys in {step} batches")
    # every key ever written, its bucket and its last-write version (= score)
    allk = gen.unique_keys(seed, 1, 0, cursor, device=dev())
    allb = cf.buckets_of(allk, cap)
    alls = torch.repeat_interleave(torch.arange(1, step + 1, dtype=torch.int64, device=dev()), 1 << 20)
    times = {"find": 0.0, "assign": 0.0, "insert_or_assign": 0.0}
    warm, steps = 5, 20
    for j in range(warm + steps):
        step += 1
        resident = cf.resident_keys(allk, alls, cap, allb)
        o = torch.argsort(allk)
        sk, sv = allk[o], alls[o]
        perm = torch.randperm(resident.numel(), device=dev())
        q = gen.shuffle(torch.cat([resident[perm[: 943718]], gen.unique_keys(seed, 2, j << 20, 104858, device=dev())]),
                        seed, 10 + j)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        out = torch.empty((q.numel(), D), dtype=torch.float32, device=dev())
        fnd = torch.empty(q.numel(), dtype=torch.uint8, device=dev())
        ak = resident[perm[943718: 943718 + (1 << 19)]]
        av = gen.values(ak, step, D)
        asc = torch.full((ak.numel(),), step, dtype=torch.int64, device=dev())
        new = gen.unique_keys(seed, 1, cursor, 1 << 17, device=dev())
        cursor += 1 << 17
        uk = gen.shuffle(torch.cat([new, resident[perm[-(1 << 17):]]]), seed, 20 + j)
        uv = gen.values(uk, step, D)
        usc = torch.full((uk.numel(),), step, dtype=torch.int64, device=dev())
        torch.cuda.synchronize()
        ev[0].record()
        tab.find(q, values_out=out, found_out=fnd)
        ev[1].record()
        tab.assign(ak, av, asc)
        ev[2].record()
        tab.insert_or_assign(uk, uv, usc)
        ev[3].record()
        torch.cuda.synchronize()
        if j >= warm:
            times["find"] += ev[0].elapsed_time(ev[1])
            times["assign"] += ev[1].elapsed_time(ev[2])
            times["insert_or_assign"] += ev[2].elapsed_time(ev[3])
        # the find saw the table before this step's writes
        idx = torch.clamp(torch.searchsorted(resident, q), max=resident.numel() - 1)
        expect = resident[idx] == q
        assert torch.equal(fnd.bool(), expect)
        ver = sv[torch.searchsorted(sk, q[expect])]
        assert torch.equal(out[expect].view(torch.int32), gen.values(q[expect], ver, D).view(torch.int32))
        # this step's writes: assigned and re-inserted keys take the step as
        # score, new keys join with it
        alls = alls.clone()
        o_all = torch.argsort(allk)
        at = o_all[torch.searchsorted(allk[o_all], torch.cat([ak, uk[~torch.isin(uk, new)]]))]
        alls[at] = step
        allk = torch.cat([allk, new])
        allb = torch.cat([allb, cf.buckets_of(new, cap)])
        alls = torch.cat([alls, torch.full((new.numel(),), step, dtype=torch.int64, device=dev())])
    k, _, s, p = export_all(tab)
    check_invariants(tab, k, p, cap)
    o = torch.argsort(allk)
    sk, sv = allk[o], alls[o]
    assert torch.equal(s, sv[torch.searchsorted(sk, k)])
    resident = cf.assert_table_matches(k, p, allk, alls, cap, allb)
    log(f"mixed: after {warm + steps} steps all {cap // SLOTS} buckets equal the closed form")
    check_find_exact(tab, gen.shuffle(resident[: 1 << 20], seed, 99), resident,
                     lambda kk: sv[torch.searchsorted(sk, kk)])
    n = {"find": 1 << 20, "assign": 1 << 19, "insert_or_assign": 1 << 18}
    log("mixed: " + ", ".join(f"{op} {n[op] * steps / ms / 1e6:.3f} B-KV/s" for op, ms in times.items())
        + f"; step {sum(times.values()) / steps:.3f} ms, {(1 << 20) * 1.75 * steps / sum(times.values()) / 1e6:.3f} B-KV/s")
    tab.close()


def test_other_calls_at_full_size():
    """find*, contains, insert_and_evict and find_or_insert on a full 2^26-slot
    dim-64 single-bucket table (the benchmark's tables and batch size). find*:
    found iff exported, address = value base + exported position * row size,
    score = last write. insert_and_evict (90 % resident, 10 % new, higher
    score): the hand-back is exactly (resident before ∪ offered) − resident
    after, each entry with the row and score of its last write.
    find_or_insert (90 % resident, 10 % new): found iff resident before, hits
    return the stored row, misses keep theirs; afterwards every resident key
    carries its last written score. After every write call every bucket
    equals the closed form, and resident keys are drawn from it."""
    H = hkv()
    cap, D, batch = 1 << 26, 64, 1 << 20
    seed = 0x484B56000000BB00
    tab = H.HashTable(cap, D)
    cursor, step = 0, 0
    parts = []
    fill = cf.FillCount(cap, dev())
    while fill.size() < cap:
        step += 1
        k = gen.unique_keys(seed, 1, cursor, batch, device=dev())
        tab.insert_or_assign(k, gen.values(k, step, D), torch.full((batch,), step, dtype=torch.int64, device=dev()))
        parts.append((batch, step))
        cursor += batch
        assert tab.size() == fill.add(k)
    allk = gen.unique_keys(seed, 1, 0, cursor, device=dev())
    alls = torch.cat([torch.full((n,), st, dtype=torch.int64, device=dev()) for n, st in parts])
    order = torch.argsort(allk)
    sk, ss = allk[order], alls[order].clone()  # last written score (= row version) of every key seen

    def last(keys):
        return ss[torch.searchsorted(sk, keys)]

    k, _, s, p = export_all(tab)
    check_invariants(tab, k, p, cap)
    ko = torch.argsort(k)
    rp = p[ko]  # positions of the exported keys in sorted key order
    rk = cf.assert_table_matches(k, p, sk, ss, cap)  # resident keys by the closed form, sorted
    assert torch.equal(rk, k[ko])
    assert torch.equal(s, last(k))
    log(f"other calls: table full after {step} batches")

    # find* and contains
    rng = torch.Generator(device="cpu").manual_seed(11)
    hits = rk[torch.randperm(rk.numel(), generator=rng)[: int(0.9 * batch)].to(dev())]
    q = gen.shuffle(torch.cat([hits, gen.unique_keys(seed, 7, 0, batch - hits.numel(), device=dev())]), seed, 3)
    ptrs = torch.full((batch,), -1, dtype=torch.int64, device=dev())
    found = torch.empty(batch, dtype=torch.uint8, device=dev())
    scores = torch.full((batch,), 0x5EED, dtype=torch.int64, device=dev())
    tab.find_ptr(q, ptrs_out=ptrs, found_out=found, scores_out=scores)
    cont = tab.contains(q)
    torch.cuda.synchronize()
    idx = torch.clamp(torch.searchsorted(rk, q), max=rk.numel() - 1)
    expect = rk[idx] == q
    assert torch.equal(found.bool(), expect) and torch.equal(cont.bool(), expect)
    assert bool((ptrs[~expect] == 0).all()) and bool((scores[~expect] == 0x5EED).all())
    assert torch.equal(scores[expect], last(q[expect]))
    base = ptrs[expect] - rp[idx[expect]] * (4 * D)
    assert bool((base == base[0]).all())
    log("other calls: find* and contains exact")

    # insert_and_evict: resident keys re-written with a higher score, new keys
    step += 1
    pre = rk
    res = rk[torch.randperm(rk.numel(), generator=rng)[: int(0.9 * batch)].to(dev())]
    new = gen.unique_keys(seed, 1, cursor, batch - res.numel(), device=dev())
    cursor += new.numel()
    uk = gen.shuffle(torch.cat([res, new]), seed, 4)
    ek, ev, es, cnt = tab.insert_and_evict(uk, gen.values(uk, step, D),
                                           torch.full((batch,), step, dtype=torch.int64, device=dev()))
    torch.cuda.synchronize()
    m = int(cnt.item())
    allk = torch.cat([sk, new])
    alls = torch.cat([ss, torch.full((new.numel(),), step, dtype=torch.int64, device=dev())])
    order = torch.argsort(allk)
    sk, ss = allk[order], alls[order].clone()
    ss[torch.searchsorted(sk, res)] = step
    k2, _, s2, p2 = export_all(tab)
    check_invariants(tab, k2, p2, cap)
    assert torch.equal(s2, last(k2))
    post = cf.assert_table_matches(k2, p2, sk, ss, cap)
    union = torch.unique(torch.cat([pre, uk]))
    gone = union[~torch.isin(union, post)]
    out = torch.sort(ek[:m]).values
    assert m == gone.numel() and torch.equal(out, gone)
    assert torch.equal(es[:m], last(ek[:m]))
    assert torch.equal(ev[:m].view(torch.int32), gen.values(ek[:m], es[:m], D).view(torch.int32))
    log(f"other calls: insert_and_evict handed back {m} entries, exact")

    # find_or_insert
    step += 1
    rk2 = post
    res = rk2[torch.randperm(rk2.numel(), generator=rng)[: int(0.9 * batch)].to(dev())]
    new = gen.unique_keys(seed, 1, cursor, batch - res.numel(), device=dev())
    uk = gen.shuffle(torch.cat([res, new]), seed, 5)
    rows = gen.values(uk, step, D)
    offered = rows.clone()
    _, fnd = tab.find_or_insert(uk, rows, torch.full((batch,), step, dtype=torch.int64, device=dev()))
    torch.cuda.synchronize()
    was = torch.isin(uk, rk2)
    assert torch.equal(fnd.bool(), was)
    assert torch.equal(rows[was].view(torch.int32), gen.values(uk[was], last(uk[was]), D).view(torch.int32))
    assert torch.equal(rows[~was], offered[~was])
    allk = torch.cat([sk, new])
    alls = torch.cat([ss, torch.full((new.numel(),), step, dtype=torch.int64, device=dev())])
    order = torch.argsort(allk)
    sk, ss = allk[order], alls[order].clone()
    ss[torch.searchsorted(sk, res)] = step  # hits take the offered score
    k3, v3, s3, p3 = export_all(tab, with_values=False)
    check_invariants(tab, k3, p3, cap)
    assert torch.equal(s3, last(k3))
    cf.assert_table_matches(k3, p3, sk, ss, cap)
    log("other calls: find_or_insert exact")
    tab.close()
