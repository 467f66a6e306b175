"""Seeded synthetic inputs for the hash-table workloads.

This module is shared by the tests, the benchmark and the smoke check, and
feeds the same arrays to the HIP library and to the CPU oracle. It holds none
of the table's arithmetic: no bucket hash, digest, probe or eviction logic.

Every generator is counter-based, so any slice of a stream can be produced
on its own, on the CPU or on a GPU, with identical bits:

* ``mix64`` is the output function of Vigna's SplitMix64 (a bijection on
  64-bit words). Keys drawn as ``mix64(counter ^ salt)`` are therefore
  distinct for distinct counters, which gives batches of unique keys without
  any deduplication.
* values are ``((r >> 40) - 2**23) * 2**-23`` for a 64-bit word ``r`` drawn
  per (key, version, column); that is uniform on [-1, 1) and exact in float32,
  so a row can be regenerated from its key and version alone.
* Zipf ranks use Hormann and Derflinger's rejection-inversion sampler (1996).

64-bit words live in ``torch.int64`` tensors holding the unsigned bit pattern
(``.numpy().view(numpy.uint64)`` gives the unsigned view).
"""

from __future__ import annotations

import math

import numpy as np
import torch

_M64 = (1 << 64) - 1
EMPTY_KEY = 0xFFFFFFFFFFFFFFFF
LOCKED_KEY = 0xFFFFFFFFFFFFFFFE

GOLDEN = 0x9E3779B97F4A7C15
_SM_M1 = 0xBF58476D1CE4E5B9
_SM_M2 = 0x94D049BB133111EB


def as_i64(x: int) -> int:
    """Unsigned 64-bit integer -> the signed value with the same bits."""
    x &= _M64
    return x - (1 << 64) if x >= (1 << 63) else x


def as_u64(x: int) -> int:
    return x & _M64


def _srl(x: torch.Tensor, n: int) -> torch.Tensor:
    """Logical right shift of int64 tensors holding unsigned bit patterns."""
    return (x >> n) & ((1 << (64 - n)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64's output function (Vigna): a bijection on 64-bit words."""
    z = (z ^ _srl(z, 30)) * as_i64(_SM_M1)
    z = (z ^ _srl(z, 27)) * as_i64(_SM_M2)
    return z ^ _srl(z, 31)


def mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _SM_M1) & _M64
    z = ((z ^ (z >> 27)) * _SM_M2) & _M64
    return z ^ (z >> 31)


def mix64_numpy(z: np.ndarray) -> np.ndarray:
    """Same function in numpy uint64 arithmetic (used to check the torch one)."""
    z = z.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_SM_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_SM_M2)
    return z ^ (z >> np.uint64(31))


def stream_salt(seed: int, stream: int) -> int:
    """64-bit salt of one named sub-stream of a master seed."""
    return mix64_int(mix64_int(seed) ^ ((stream * GOLDEN) & _M64))


def counter_words(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """``mix64(counter ^ salt)`` for counters start .. start+count-1."""
    c = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return mix64(c ^ as_i64(stream_salt(seed, stream)))


def unique_keys(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Uniform 64-bit keys, distinct across every (start, count) slice of one
    (seed, stream). Different streams of one seed are disjoint when their
    counter ranges are disjoint: stream s draws counters from [s*2^40, (s+1)*2^40)."""
    base = stream << 40
    if start < 0 or start + count > (1 << 40):
        raise ValueError("counter range outside the stream")
    keys = counter_words(seed, 0, base + start, count, device)
    if bool(((keys == -1) | (keys == -2)).any()):
        raise RuntimeError("a generated key hit a reserved value; pick another seed")
    return keys


def keys_in_range(seed: int, stream: int, count: int, lo: int, hi: int, device="cpu",
                  distinct: bool = True) -> torch.Tensor:
    """``count`` keys uniform on [lo, hi), distinct within the batch when asked
    (draws extra words and keeps the first occurrences, input order preserved)."""
    span = hi - lo
    assert 0 < span < (1 << 62)
    extra = 0
    while True:
        n = count + extra + 64
        w = counter_words(seed, stream, 0, n, device)
        k = lo + (_srl(w, 1) % span)
        if not distinct:
            return k[:count]
        kc = k.cpu().numpy()
        _, first = np.unique(kc, return_index=True)
        first.sort()
        if first.size >= count:
            return k[torch.from_numpy(first[:count]).to(k.device)]
        extra = 2 * extra + count // 8 + 64


def values(keys: torch.Tensor, version, dim: int, seed: int = 0) -> torch.Tensor:
    """Row of ``dim`` float32 values per key, exact, uniform on [-1, 1).

    ``version`` is an int or an int64 tensor (one per key); a row is fully
    determined by (seed, key, version)."""
    n = keys.numel()
    dev = keys.device
    if not torch.is_tensor(version):
        version = torch.full((n,), as_i64(version), dtype=torch.int64, device=dev)
    version = version.to(device=dev, dtype=torch.int64)
    base = mix64(mix64(keys.to(torch.int64) ^ as_i64(stream_salt(seed, 0x5A1))) ^ version)
    col = (torch.arange(1, dim + 1, dtype=torch.int64, device=dev) * as_i64(GOLDEN)).view(1, dim)
    r = mix64(base.view(n, 1) + col)
    q = _srl(r, 40) - (1 << 23)
    return q.to(torch.float32) * (1.0 / (1 << 23))


def shuffle(x: torch.Tensor, seed: int, stream: int) -> torch.Tensor:
    """Seeded permutation (sort by counter words)."""
    w = counter_words(seed, stream, 0, x.numel(), x.device)
    return x[torch.argsort(w)]


def uniform01(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """float64 uniform on [0, 1) with 53 random bits per draw."""
    w = counter_words(seed, stream, start, count, device)
    return _srl(w, 11).to(torch.float64) * (1.0 / (1 << 53))


class Zipf:
    """Rejection-inversion sampler of Hormann and Derflinger (1996) for
    P(k) proportional to k^-alpha on {1, ..., n}, vectorised over a batch.

    ``draw(seed, stream, start, count)`` uses one uniform per attempt taken
    from counter ranges, so a batch is a pure function of its arguments."""

    def __init__(self, alpha: float, n: int):
        assert alpha > 0 and n >= 1
        self.a = float(alpha)
        self.n = int(n)
        self.h_x1 = self._H(1.5) - 1.0
        self.h_n = self._H(self.n + 0.5)
        self.s = 2.0 - self._Hinv(self._H(2.5) - self._h(2.0))

    def _h(self, x):
        return math.exp(-self.a * math.log(x))

    def _H(self, x):  # integral of h, shifted so that it is well defined at a = 1
        lx = math.log(x)
        return self._helper2((1.0 - self.a) * lx) * lx

    def _Hinv(self, x):
        t = max(x * (1.0 - self.a), -1.0)
        return math.exp(self._helper1(t) * x)

    @staticmethod
    def _helper1(x):  # log(1 + x) / x
        return math.log1p(x) / x if abs(x) > 1e-8 else 1.0 - x * (0.5 - x * (1.0 / 3.0 - 0.25 * x))

    @staticmethod
    def _helper2(x):  # (exp(x) - 1) / x
        return math.expm1(x) / x if abs(x) > 1e-8 else 1.0 + x * 0.5 * (1.0 + x / 3.0 * (1.0 + 0.25 * x))

    # Vectorised forms of the helpers.
    def _t_h(self, x):
        return torch.exp(-self.a * torch.log(x))

    def _t_H(self, x):
        lx = torch.log(x)
        y = (1.0 - self.a) * lx
        small = y.abs() <= 1e-8
        ys = torch.where(small, torch.ones_like(y), y)
        h2 = torch.where(small, 1.0 + y * 0.5 * (1.0 + y / 3.0 * (1.0 + 0.25 * y)), torch.expm1(ys) / ys)
        return h2 * lx

    def _t_Hinv(self, x):
        t = torch.clamp(x * (1.0 - self.a), min=-1.0)
        small = t.abs() <= 1e-8
        ts = torch.where(small, torch.ones_like(t), t)
        h1 = torch.where(small, 1.0 - t * (0.5 - t * (1.0 / 3.0 - 0.25 * t)), torch.log1p(ts) / ts)
        return torch.exp(h1 * x)

    def draw(self, seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
        """Ranks for draws start .. start+count-1 of one (seed, stream)."""
        out = torch.zeros(count, dtype=torch.int64, device=device)
        pending = torch.arange(count, dtype=torch.int64, device=device)
        salt = as_i64(stream_salt(seed, stream))
        attempt = 0
        while pending.numel() > 0:
            # attempt a of draw i uses counter (start + i) * 64 + a
            w = mix64(((start + pending) * 64 + attempt) ^ salt)
            u01 = _srl(w, 11).to(torch.float64) * (1.0 / (1 << 53))
            u = self.h_n + u01 * (self.h_x1 - self.h_n)
            x = self._t_Hinv(u)
            k = torch.clamp(torch.floor(x + 0.5), 1, self.n)
            accept = (k - x <= self.s) | (u >= self._t_H(k + 0.5) - self._t_h(k))
            out[pending[accept]] = k[accept].to(torch.int64)
            pending = pending[~accept]
            attempt += 1
            if attempt >= 64:
                raise RuntimeError("Zipf sampler did not converge")
        return out
