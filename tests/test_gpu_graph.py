"""Calls captured into a HIP graph and replayed (the way launch-bound small
batches avoid per-call launch costs). Capture works when every call of the
table is issued on the capturing stream (a table used from one stream records
no events) and the inserter workspace was sized by an eager call of the same
batch size before capture (capture cannot allocate). Every replay is checked
against the oracle, with eager work (inserts among it) and synchronizations
between replays."""

import numpy as np
import pytest
import torch

import hkv_inputs as gen
import oracle
from conftest import gpu_available
from helpers import SLOTS
from test_gpu_parity import assert_same_contents, dev, hkv, np_u64, sample_present, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_find_and_insert_or_assign_replay_from_a_graph():
    H = hkv()
    C, D, n = 64 * SLOTS, 16, 4096
    seed = 0x484B56000000C4A9
    s = torch.cuda.Stream()
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    qk = torch.empty(n, dtype=torch.int64, device=dev())
    out = torch.empty((n, D), dtype=torch.float32, device=dev())
    found = torch.empty(n, dtype=torch.uint8, device=dev())
    uk = torch.empty(n, dtype=torch.int64, device=dev())
    uv = torch.empty((n, D), dtype=torch.float32, device=dev())
    us = torch.empty(n, dtype=torch.int64, device=dev())
    with torch.cuda.stream(s):
        step = 0
        for j in range(3):  # eager fill on the capturing stream (sizes the workspace for n keys)
            step += 1
            k = gen.unique_keys(seed, 1, j * n, n, device=dev())
            v = gen.values(k, step, D)
            sc = torch.full((n,), step, dtype=torch.int64, device=dev())
            tab.insert_or_assign(k, v, sc, stream=s)
            o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            tab.find(qk, values_out=out, found_out=found, stream=s)
            tab.insert_or_assign(uk, uv, us, stream=s)
        cursor = 3 * n
        for r in range(4):
            step += 1
            # inputs of this replay, written eagerly into the captured buffers
            hits = sample_present(o, n // 2, 100 + r)
            q = np.concatenate([hits, np_u64(gen.unique_keys(seed, 2, r * n, n - hits.size))])
            qk.copy_(to_dev(q))
            res = sample_present(o, n // 4, 200 + r)
            new = np_u64(gen.unique_keys(seed, 1, cursor, n - res.size))
            cursor += new.size
            u = np.concatenate([res, new])
            uk.copy_(to_dev(u))
            uv.copy_(gen.values(uk, step, D))
            us.fill_(step)
            out.fill_(0.0)
            found.fill_(7)
            g.replay()
            s.synchronize()
            # find saw the table before this replay's insert_or_assign
            ov, of, _, _ = o.find(q)
            assert np.array_equal(found.cpu().numpy(), of)
            hit = of.astype(bool)
            assert np.array_equal(out.cpu().numpy()[hit].view(np.uint32), ov[hit].view(np.uint32))
            o.insert_or_assign(u, np.full(n, step, np.uint64), values=uv.cpu().numpy())
            assert_same_contents(tab, o)
            if r % 2 == 0:
                # an eager insert between replays: eager calls tag the chain
                # heads with a fresh epoch, replays run at the captured one
                step += 1
                e_res = sample_present(o, n // 4, 300 + r)
                e_new = np_u64(gen.unique_keys(seed, 1, cursor, n - e_res.size))
                cursor += e_new.size
                ek = to_dev(np.concatenate([e_res, e_new]))
                ev = gen.values(ek, step, D)
                es = torch.full((n,), step, dtype=torch.int64, device=dev())
                tab.insert_or_assign(ek, ev, es, stream=s)
                s.synchronize()
                o.insert_or_assign(np_u64(ek), np_u64(es), values=ev.cpu().numpy())
                assert_same_contents(tab, o)
    tab.close()


def _graph_batches(o, n, r, cursor, seed, D, step):
    """A replay's insert batch: a quarter resident keys, the rest new."""
    res = sample_present(o, n // 4, 500 + r)
    new = np_u64(gen.unique_keys(seed, 1, cursor, n - res.size))
    return np.concatenate([res, new]), cursor + new.size


def test_captured_insert_with_outcome_counts():
    """insert_or_assign captured with the outcome counters on: every replay
    leaves the oracle's contents and adds that call's counts (set
    differences of the oracle's states before and after)."""
    H = hkv()
    C, D, n = 32 * SLOTS, 8, 2048
    seed = 0x484B56000000C4AA
    s = torch.cuda.Stream()
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    uk = torch.empty(n, dtype=torch.int64, device=dev())
    uv = torch.empty((n, D), dtype=torch.float32, device=dev())
    us = torch.empty(n, dtype=torch.int64, device=dev())
    with torch.cuda.stream(s):
        step, cursor = 0, 0
        for j in range(2):  # eager fill (sizes the workspace for n keys)
            step += 1
            k = gen.unique_keys(seed, 1, cursor, n, device=dev())
            cursor += n
            v = gen.values(k, step, D)
            sc = torch.full((n,), step, dtype=torch.int64, device=dev())
            tab.insert_or_assign(k, v, sc, stream=s)
            o.insert_or_assign(np_u64(k), np_u64(sc), values=v.cpu().numpy())
        s.synchronize()
        tab.count_outcomes()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            tab.insert_or_assign(uk, uv, us, stream=s)
        was = tab.outcomes()
        for r in range(3):
            step += 1
            u, cursor = _graph_batches(o, n, r, cursor, seed, D, step)
            before = set(o.export()["keys"].tolist())
            uk.copy_(to_dev(u))
            uv.copy_(gen.values(uk, step, D))
            us.fill_(step)
            g.replay()
            s.synchronize()
            o.insert_or_assign(u, np.full(n, step, np.uint64), values=uv.cpu().numpy())
            assert_same_contents(tab, o)
            after = set(o.export()["keys"].tolist())
            b = set(u.tolist())
            now = tab.outcomes()
            assert {k: now[k] - was[k] for k in now} == {
                "updated": len(b & before), "inserted": len(after - before),
                "evicted": len(before - after), "rejected": len(b - before - after)}
            was = now
    tab.close()


def test_noalloc_insert_replays_from_a_graph():
    """The entry point that allocates nothing, captured with no eager
    inserter call before it (it needs no workspace) and replayed four times
    with fresh inputs, each replay equal to the oracle."""
    from hash_table_cache_amd import _native

    H = hkv()
    C, D, n = 32 * SLOTS, 16, 2048
    seed = 0x484B56000000C4AB
    s = torch.cuda.Stream()
    tab = H.HashTable(C, D)
    o = oracle.OracleTable(C, D)
    uk = torch.empty(n, dtype=torch.int64, device=dev())
    uv = torch.empty((n, D), dtype=torch.float32, device=dev())
    us = torch.empty(n, dtype=torch.int64, device=dev())
    L = _native.load()
    with torch.cuda.stream(s):
        uk.zero_()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            st = L.hkv_insert_or_assign_noalloc(tab.handle, n, uk.data_ptr(), uv.data_ptr(), us.data_ptr(),
                                                s.cuda_stream)
        assert st == _native.HKV_OK, L.hkv_last_error().decode()
        step, cursor = 0, 0
        for r in range(4):
            step += 1
            u, cursor = _graph_batches(o, n, r, cursor, seed, D, step)
            uk.copy_(to_dev(u))
            uv.copy_(gen.values(uk, step, D))
            us.fill_(step)
            g.replay()
            s.synchronize()
            o.insert_or_assign(u, np.full(n, step, np.uint64), values=uv.cpu().numpy())
            assert_same_contents(tab, o)
    tab.close()
