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
