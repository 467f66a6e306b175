"""The seeded input generators: bit-identical across backends, unique keys,
exact values on [-1, 1), Zipf frequencies."""

import numpy as np
import torch

import hkv_inputs as gen


def test_mix64_torch_matches_numpy():
    z = torch.arange(-5000, 5000, dtype=torch.int64) * 0x9E3779B97F4A7C1
    a = gen.mix64(z).numpy().view(np.uint64)
    b = gen.mix64_numpy(z.numpy().view(np.uint64))
    assert np.array_equal(a, b)
    assert gen.mix64_int(12345) == int(gen.mix64(torch.tensor([12345])).numpy().view(np.uint64)[0])


def test_unique_keys_distinct_and_streams_disjoint():
    a = gen.unique_keys(1, 0, 0, 200000)
    b = gen.unique_keys(1, 1, 0, 200000)
    c = gen.unique_keys(1, 0, 200000, 1000)
    allk = torch.cat([a, b, c])
    assert torch.unique(allk).numel() == allk.numel()
    assert torch.equal(gen.unique_keys(1, 0, 5, 10), a[5:15])


def test_keys_in_range_distinct_in_range():
    k = gen.keys_in_range(9, 1, 20000, 1, 1 << 40).numpy()
    assert np.unique(k).size == k.size
    assert k.min() >= 1 and k.max() < (1 << 40)


def test_values_exact_and_regenerable():
    k = gen.unique_keys(2, 0, 0, 1000)
    v = gen.values(k, 17, 33)
    assert v.dtype == torch.float32 and v.shape == (1000, 33)
    assert float(v.min()) >= -1.0 and float(v.max()) < 1.0
    q = (v.double() * (1 << 23))
    assert torch.equal(q, torch.round(q))  # multiples of 2^-23: exact in fp32
    assert torch.equal(gen.values(k[10:20], 17, 33), v[10:20])
    assert not torch.equal(gen.values(k, 18, 33), v)
    ver = torch.arange(1000, dtype=torch.int64)
    assert torch.equal(gen.values(k[3:4], 3, 33), gen.values(k, ver, 33)[3:4])


def test_zipf_frequencies():
    n, alpha = 50, 1.05
    z = gen.Zipf(alpha, n)
    r = z.draw(4, 1, 0, 400000).numpy()
    assert r.min() >= 1 and r.max() <= n
    p = np.arange(1, n + 1, dtype=np.float64) ** -alpha
    p /= p.sum()
    counts = np.bincount(r, minlength=n + 1)[1:]
    exp = p * r.size
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < (n - 1) + 6 * np.sqrt(2 * (n - 1))
    assert torch.equal(z.draw(4, 1, 100, 50), torch.from_numpy(r[100:150]))
