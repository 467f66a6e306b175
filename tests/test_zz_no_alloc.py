"""The entry point that allocates nothing, hkv_insert_or_assign_noalloc,
called through the C ABI, against hkv_insert_or_assign: the same batches,
applied to two tables of the same shape, one through each entry point, must
leave the same contents after every call - two calls in a row, the second
with a smaller batch - exactly (keys per bucket, rows and scores bit for
bit) in single-bucket mode and, in dual-bucket mode below the first
eviction, as sets of (key, row, score). Oversized batches are refused."""

import ctypes

import numpy as np
import pytest
import torch

import hkv_inputs as gen
from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SLOTS = 128


def dev():
    return torch.device("cuda", 0)


def noalloc(tab, keys, values, scores):
    from hash_table_cache_amd import _native

    L = _native.load()
    st = L.hkv_insert_or_assign_noalloc(tab.handle, keys.numel(), keys.data_ptr(), values.data_ptr(),
                                        scores.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == _native.HKV_OK, L.hkv_last_error().decode()


def contents(tab):
    k, v, s, p = tab.export_batch()
    o = torch.argsort(k)
    return k[o], v[o], s[o], torch.div(p[o], SLOTS, rounding_mode="floor")


def assert_same(a, b, same_buckets):
    ka, va, sa, ba = contents(a)
    kb, vb, sb, bb = contents(b)
    assert torch.equal(ka, kb)
    assert torch.equal(va.view(torch.int32), vb.view(torch.int32))
    assert torch.equal(sa, sb)
    if same_buckets:
        assert torch.equal(ba, bb)
    return ka.numel()


@pytest.mark.parametrize("dual", [False, True])
def test_noalloc_matches_insert_or_assign(dual):
    import hash_table_cache_amd as H

    C, D = 1 << 16, 32
    a = H.HashTable(C, D, dual_bucket=dual)
    b = H.HashTable(C, D, dual_bucket=dual)
    seed = 0x484B5600000077 + int(dual)
    # a common start: both tables a quarter full through insert_or_assign
    k0 = gen.unique_keys(seed, 1, 0, C // 4, device=dev())
    s0 = torch.ones(k0.numel(), dtype=torch.int64, device=dev())
    for t in (a, b):
        t.insert_or_assign(k0, gen.values(k0, 1, D), s0)
    # two calls in a row, the second smaller: resident keys re-written plus new
    # keys (single-bucket mode fills past capacity, so buckets also evict)
    sizes = [(C // 2, 3 * C // 4 if not dual else C // 8), (C // 16, 1000)]
    cursor = C // 4
    for step, (n_res, n_new) in enumerate(sizes, start=2):
        res = k0[torch.randperm(k0.numel(), device=dev())[:n_res]]
        new = gen.unique_keys(seed, 1, cursor, n_new, device=dev())
        cursor += n_new
        k = gen.shuffle(torch.cat([res, new]), seed, step)
        v = gen.values(k, step, D)
        sc = torch.full((k.numel(),), step, dtype=torch.int64, device=dev())
        a.insert_or_assign(k, v, sc)
        noalloc(b, k, v, sc)
        torch.cuda.synchronize()
        n = assert_same(a, b, same_buckets=not dual)
        assert a.size() == b.size() == n
    a.close()
    b.close()


def test_noalloc_refuses_an_oversized_batch():
    import hash_table_cache_amd as H
    from hash_table_cache_amd import _native

    tab = H.HashTable(1 << 12, 4)
    n = _native.NOALLOC_MAX_KEYS + 1
    k = torch.zeros(n, dtype=torch.int64, device=dev())
    v = torch.zeros((n, 4), dtype=torch.float32, device=dev())
    L = _native.load()
    st = L.hkv_insert_or_assign_noalloc(tab.handle, n, k.data_ptr(), v.data_ptr(), k.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == _native.HKV_EINVAL
    assert "exceeds its limit" in L.hkv_last_error().decode()
    assert tab.size() == 0
    tab.close()
