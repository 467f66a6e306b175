"""Find / upsert throughput of the cache-semantic hash table on one MI355X.

Workload (defaults): four single-bucket tables of 2^26 slots with dim-64
float32 rows, pre-filled with uniform distinct 64-bit keys (score = batch
counter) to load factors 0.50, 0.75, 0.90 and 1.00. One step issues, on each
table, a find of 2^20 keys (90 % resident, 10 % never inserted) followed by an
insert_or_assign of 2^20 keys (90 % resident keys refreshed with new rows and
the current step as score, 10 % new keys). The steps of each phase run table
by table (every step on the 0.50 table, then on the 0.75 table, ...), as the
paper measures each load factor on its own table; --interleave-tables runs
them step by step across the tables. Inputs are generated on the GPU before
the timed region. value = keys processed by all calls / wall time.

The K timed steps issue nothing but the calls. They are followed by K more
steps of the same workload in which every kernel launch is timed with a pair
of HIP events that the kernel's own dispatch records (the library launches
with hipExtLaunchKernelGGL while hkv_profile_start/stop is on; this adds
about 6 % to a step, so it stays out of the value); the kernel with the
largest total time is the dominant one and gets the roofline figure:
algorithmic bytes per launch / average launch time, against 8 TB/s.
Per-lambda call times are the table's kernel times per call.
Algorithmic bytes per key (D = dim, h = hit fraction, f = resident fraction
of an upsert batch, e = fraction of new keys that evict, i.e. land in a full
bucket):
  find          8 key + 128 digest line + 4 false-positive keys (0.5 x 8)
                + h (8 key + 4D row read + 4D row write) + 1 found flag
  upsert_probe  8 key + 128 digest line + 4 false-positive keys
                + f (8 key + 4D row in + 8 score in + 4D row write + 8 score write)
                + (1 - f) 8 (chain link: head exchange + next)
  upsert_owner  4 next (every key) + (1 - f) [8 key + 8 score + 4D row in
                + 4 head + 4 occ + 128 digest line + 4 false-positive keys
                + 8 key + 1 digest + 8 score + 4D row write
                + e (1024 score column + 8 tied key)]

Prints one JSON line. --gpus N > 1 exits: the table lives on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "find & upsert B-KV/s at λ=0.5–1.0, dim=64 fp32; % of HBM BW peak"
HBM_PEAK_GBS = 8000.0
SEED = 0x484B560000000002


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--dim", type=int, default=64)
    p.add_argument("--capacity-log2", type=int, default=26)
    p.add_argument("--batch-log2", type=int, default=20)
    p.add_argument("--lambdas", default="0.5,0.75,0.9,1.0")
    p.add_argument("--hit-frac", type=float, default=0.9)
    p.add_argument("--new-frac", type=float, default=0.1, help="fraction of new keys in each upsert batch")
    p.add_argument("--hit-pool", choices=("resident", "recent"), default="resident",
                   help="where the resident keys of the find and upsert batches come from: sampled uniformly "
                        "from the whole resident set (default), or from the 2*batch most recently inserted keys "
                        "(a recency-skewed mix whose key lines partly stay in the Infinity Cache)")
    p.add_argument("--unique-keys", action="store_true",
                   help="create the tables with HKV_FLAG_UNIQUE_KEYS (every write batch is distinct by construction)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=6,
                   help="timed steps of the first table that the CPU oracle baseline replays")
    p.add_argument("--insert-steps", type=int, default=5,
                   help="extra all-new-key insert batches on the full table, reported in detail")
    p.add_argument("--find-only", action="store_true", help="time find batches only")
    p.add_argument("--interleave-tables", action="store_true",
                   help="run each step across all load-factor tables instead of table by table")
    p.add_argument("--no-extra-ops", dest="extra_ops", action="store_false",
                   help="skip the find*/contains/insert_and_evict/find_or_insert measurements")
    p.add_argument("--capacity-sweep", default="", metavar="LOG2S",
                   help="only measure find on full tables of these capacities (e.g. 24,26,28) and exit")
    p.add_argument("--mixed", default="", metavar="MIXES",
                   help="concurrency ablation over these thread mixes, e.g. " + ",".join(MIXES))
    p.add_argument("--mixed-batches", type=int, default=200, help="batches per thread in --mixed")
    p.add_argument("--api-sweep", action="store_true",
                   help="every call on the pure-HBM configurations A-C (at --api-lambdas)")
    p.add_argument("--api-lambdas", default="0.5", help="load factors of --api-sweep, e.g. 0.5,0.75,1.0")
    p.add_argument("--online", action="store_true",
                   help="single- vs dual-bucket continuous Zipf upsert at full capacity (use --capacity-log2 27)")
    p.add_argument("--online-modes", default="single,dual", help="bucket modes of --online")
    p.add_argument("--graph", action="store_true",
                   help="small launch-bound batches issued eagerly and replayed from a HIP graph")
    p.add_argument("--triple", action="store_true",
                   help="the mixed find/assign/insert_or_assign workload (use with --capacity-log2 27)")
    p.add_argument("--tiered", action="store_true",
                   help="the tiered-values workload (use with --capacity-log2 28 --dim 128)")
    p.add_argument("--hybrid", default="", metavar="FRACS",
                   help="value-placement sweep at these HBM fractions of the value rows, e.g. 1.0,0.5,0.0")
    p.add_argument("--cold-runs", type=int, default=0, metavar="K",
                   help="run the lambda sweep K times, each in a fresh process with fresh tables, and report "
                        "the per-lambda medians (the paper's statistic: median of cold-start runs)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB 10 times (counter calibration) and exit")
    return p.parse_args()


PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCE = os.path.join(ROOT, "hash_table_cache_amd", "csrc", "hkv_kernels.hip")
PROFILE_NAMES = {"find": "find_kernel", "upsert_probe": "upsert_probe_kernel", "upsert_owner": "upsert_owner_kernel"}


def kernel_code_sha256() -> str:
    """sha256 of the kernel source with comments and white space removed: a
    profile stays valid across comment edits, not across code changes."""
    import hashlib
    import re

    src = open(KERNEL_SOURCE, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return hashlib.sha256("".join(src.split()).encode()).hexdigest()


def profiled_traffic(kernel: str, dim: int, capacity_log2: int):
    """Bytes per launch of `kernel` between the L2s and the data fabric
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counters;
    Infinity Cache hits included) from a committed rocprofv3 summary of
    this workload, or None when no summary matches the current kernel code."""
    import glob

    sha = kernel_code_sha256()
    for path in sorted(glob.glob(os.path.join(PROFILE_DIR, "*.txt"))):
        fields = {}
        traffic = {}
        for line in open(path):
            parts = line.split()
            if len(parts) >= 2 and parts[0] in ("kernel_code_sha256", "workload_dim", "workload_capacity_log2"):
                fields[parts[0]] = parts[1]
            elif len(parts) == 3 and parts[0] == "traffic_bytes_per_launch":
                traffic[parts[1]] = int(parts[2])
        if (fields.get("kernel_code_sha256") == sha and fields.get("workload_dim") == str(dim)
                and fields.get("workload_capacity_log2") == str(capacity_log2)
                and PROFILE_NAMES.get(kernel) in traffic):
            return traffic[PROFILE_NAMES[kernel]]
    return None


def find_bytes_per_key(dim: int, h: float) -> float:
    return 8 + 128 + 4 + h * (8 + 8 * dim) + 1


def probe_bytes_per_key(dim: int, f: float) -> float:
    return 8 + 128 + 4 + f * (8 + 8 * dim + 16) + (1 - f) * 8


def owner_bytes_per_key(dim: int, f: float, e: float) -> float:
    return 4 + (1 - f) * (8 + 8 + 4 * dim + 4 + 4 + 128 + 4 + 8 + 1 + 8 + 4 * dim + e * (1024 + 8))


def launch_cv(stat) -> float:
    """Coefficient of variation of a kernel's launch times from the library's
    (launches, total, max, min, sum of squares, median) record."""
    n, tot, _, _, sq = stat[:5]
    mean = tot / n
    var = max(0.0, sq / n - mean * mean)
    return round(var ** 0.5 / mean, 4) if mean > 0 else 0.0


def batch_size(args) -> int:
    return 1 << args.batch_log2


def locate_bytes_per_key(h: float, with_ptr: bool) -> float:
    """find* / contains: 8 key + 128 digest line + 4 false-positive keys
    + h 8 key + 1 found flag (+ 8 address for find*)."""
    return 8 + 128 + 4 + h * 8 + 1 + (8 if with_ptr else 0)


def copy_bandwidth(mib: int = 2048, reps: int = 10) -> float:
    """Device-to-device copy rate (read + write bytes / s) on this GPU: the
    streaming bandwidth the hash-table kernels are compared against."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


PATTERN_SOURCE = os.path.join(ROOT, "bench_pattern_ceiling.hip")
PATTERN_EXE = os.path.join(ROOT, "_build", "bench_pattern_ceiling")


def build_pattern_ceiling() -> str:
    """Compiles the access-pattern ceiling program (a stand-alone benchmark
    of find's and the upsert probe's memory accesses, no table involved) with
    hipcc for gfx950, beside the other build products. Returns its path."""
    import pathlib

    hb = _load_build_module()
    os.makedirs(os.path.dirname(PATTERN_EXE), exist_ok=True)
    tmp = PATTERN_EXE + ".tmp"
    flags = [f for f in hb.compile_flags() if f != "-fvisibility=hidden"]
    subprocess.run([hb.hipcc(), *flags, "-x", "hip", PATTERN_SOURCE, "-o", tmp], check=True)
    pathlib.Path(tmp).replace(PATTERN_EXE)
    return PATTERN_EXE


def _load_build_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "hkv_build", os.path.join(ROOT, "hash_table_cache_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def pattern_ceiling(dim: int = 64):
    """Runs the access-pattern ceiling program (find's memory accesses on a
    2^26-slot table with rows of `dim` floats, without its arithmetic, with
    and without the chain of dependent loads) in a child process; returns its
    JSON, or None when the program has not been built."""
    if not os.path.exists(PATTERN_EXE):
        return None
    try:
        r = subprocess.run([PATTERN_EXE, str(dim)], capture_output=True, text=True, timeout=120, check=True)
        return json.loads(r.stdout)
    except (subprocess.SubprocessError, ValueError) as e:
        log(f"pattern ceiling program failed: {e}")
        return None


def calibrate_copy(mib: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "copy_GBps": 2 * n * 4 / dt / 1e9}), flush=True)


def capacity_sweep(args) -> None:
    """find on full single-bucket tables of several capacities: 2 warm-up and
    10 timed 2^20-key batches (90 % resident) per capacity, kernel time from
    the library's events. Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    dim, batch = args.dim, 1 << args.batch_log2
    out = {}
    for lg in [int(x) for x in args.capacity_sweep.split(",")]:
        cap = 1 << lg
        tab = H.HashTable(cap, dim)
        cursor, step = 0, 0
        while tab.size() < cap:
            step += 1
            k = gen.unique_keys(SEED, 70 + lg, cursor, batch, device=dev)
            cursor += batch
            tab.insert_or_assign(k, gen.values(k, step, dim, SEED), torch.full((batch,), step, dtype=torch.int64,
                                                                              device=dev))
        pool = gen.unique_keys(SEED, 70 + lg, cursor - 4 * batch, 4 * batch, device=dev)
        n_hit = int(round(batch * args.hit_frac))
        qs = []
        for j in range(12):
            perm = torch.argsort(gen.counter_words(SEED, 130 + lg, j * pool.numel(), pool.numel(), dev))
            q = torch.cat([pool[perm[:n_hit]], gen.unique_keys(SEED, 110 + lg, j * batch, batch - n_hit, device=dev)])
            qs.append(gen.shuffle(q, SEED, 150 + j))
        vals = torch.empty((batch, dim), dtype=torch.float32, device=dev)
        found = torch.empty(batch, dtype=torch.uint8, device=dev)
        for q in qs[:2]:
            tab.find(q, values_out=vals, found_out=found)
        torch.cuda.synchronize()
        tab.profile_start()
        for q in qs[2:]:
            tab.find(q, values_out=vals, found_out=found)
        ms = tab.profile_stop()["find"]
        avg = ms[1] / ms[0]
        out[f"2^{lg}"] = dict(find_ms=round(avg, 5), find_bkvs=round(batch / avg / 1e6, 3),
                              frac=round(batch * find_bytes_per_key(dim, n_hit / batch) / (avg * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4))
        log(f"capacity 2^{lg}: {out[f'2^{lg}']}")
        tab.close()
        torch.cuda.empty_cache()
    b = [v["find_bkvs"] for v in out.values()]
    print(json.dumps({"capacity_sweep": out, "dim": dim, "variation": round((max(b) - min(b)) / max(b), 4)}),
          flush=True)


def hybrid_sweep(args) -> None:
    """Value placement (the HBM watermark): full single-bucket tables of
    2^capacity_log2 slots whose value rows are all in HBM, half in HBM and half
    in pinned host memory, or all on the host. Per placement: find*, contains
    and find (value copy) on 2^batch_log2-key batches, 90 % resident; 2 warm-up
    and 10 timed batches, library event times. Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap, dim, batch = 1 << args.capacity_log2, args.dim, 1 << args.batch_log2
    row = 4 * dim
    n_hit = int(round(batch * args.hit_frac))
    out = {}
    for frac in [float(x) for x in args.hybrid.split(",")]:
        t0 = time.perf_counter()
        tab = H.HashTable(cap, dim, values_on_host=frac < 1.0, hbm_value_bytes=int(frac * cap * row))
        cursor, step = 0, 0
        while tab.size() < cap:
            step += 1
            k = gen.unique_keys(SEED, 80, cursor, batch, device=dev)
            cursor += batch
            tab.insert_or_assign(k, gen.values(k, step, dim, SEED),
                                 torch.full((batch,), step, dtype=torch.int64, device=dev))
        pool = gen.unique_keys(SEED, 80, cursor - 2 * batch, 2 * batch, device=dev)
        qs = []
        for j in range(12):
            perm = torch.argsort(gen.counter_words(SEED, 180, j * pool.numel(), pool.numel(), dev))
            q = torch.cat([pool[perm[:n_hit]], gen.unique_keys(SEED, 181, j * batch, batch - n_hit, device=dev)])
            qs.append(gen.shuffle(q, SEED, 190 + j))
        vals = torch.empty((batch, dim), dtype=torch.float32, device=dev)
        found = torch.empty(batch, dtype=torch.uint8, device=dev)
        ptrs = torch.empty(batch, dtype=torch.int64, device=dev)
        r = dict(fill_s=round(time.perf_counter() - t0, 1))
        for name in ("find_ptr", "contains", "find"):
            call = {"find_ptr": lambda q: tab.find_ptr(q, ptrs, found),
                    "contains": lambda q: tab.contains(q, found),
                    "find": lambda q: tab.find(q, vals, found)}[name]
            for q in qs[:2]:
                call(q)
            torch.cuda.synchronize()
            tab.profile_start()
            for q in qs[2:]:
                call(q)
            st = tab.profile_stop()[name]
            avg = st[1] / st[0]
            r[name] = dict(kernel_avg_ms=round(avg, 5), bkvs=round(batch / avg / 1e6, 3))
        if frac < 1.0:
            r["host_link_GBps_find"] = round(batch * args.hit_frac * (1 - frac) * row / (r["find"]["kernel_avg_ms"]
                                                                                       * 1e-3) / 1e9, 1)
        out[f"hbm_fraction_{frac}"] = r
        log(f"hbm fraction {frac}: {r}")
        tab.close()
        torch.cuda.empty_cache()
    base = out.get("hbm_fraction_1.0")
    if base:
        for k, r in out.items():
            r["find_ptr_retained"] = round(r["find_ptr"]["bkvs"] / base["find_ptr"]["bkvs"], 4)
    print(json.dumps({"hybrid": out, "capacity": cap, "dim": dim, "batch": batch, "hit_frac": args.hit_frac}),
          flush=True)


def tiered_run(args) -> None:
    """The tiered-values workload: dual-bucket table of 2^capacity_log2 slots
    (2^28 in the paper's largest configuration) with dim --dim rows (128) in
    pinned, GPU-mapped host memory. Warm cache: ranks 1 .. capacity * 17/16
    inserted coldest first in 2^19-key batches, score = batch (LRU). Each step:
    find 2^20 Zipf(1.2) draws over 2^32 ids (key = rank, not deduplicated),
    then insert_or_assign of 2^19 draws (deduplicated), score = step;
    --warmup + --steps steps, kernel times from the library's events. Prints
    one JSON line: rates per call, hit rate, key-side HBM bytes/s of find and
    the rate at which it delivers rows (a hot key's row counted at each of
    its draws), distinct keys per batch."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap, dim = 1 << args.capacity_log2, args.dim
    row = 4 * dim
    t0 = time.perf_counter()
    tab = H.HashTable(cap, dim, dual_bucket=True, values_on_host=True)
    step = 0
    hi = cap + cap // 16
    while hi > 0:
        step += 1
        lo = max(1, hi - (1 << 19) + 1)
        k = torch.arange(hi, lo - 1, -1, dtype=torch.int64, device=dev)
        hi = lo - 1
        tab.insert_or_assign(k, gen.values(k, step, dim, SEED), torch.full((k.numel(),), step, dtype=torch.int64,
                                                                          device=dev))
    torch.cuda.synchronize()
    log(f"tiered: warm table size {tab.size()} after {step} batches, {time.perf_counter() - t0:.1f}s")
    zipf = gen.Zipf(1.2, 1 << 32)
    nsteps = args.warmup + args.steps
    finds = [zipf.draw(SEED, 1, j * (1 << 20), 1 << 20, device=dev) for j in range(nsteps)]
    ups = []
    for j in range(nsteps):
        u = torch.unique(zipf.draw(SEED, 2, j * (1 << 19), 1 << 19, device=dev))
        ups.append((u, gen.values(u, step + 1 + j, dim, SEED),
                    torch.full((u.numel(),), step + 1 + j, dtype=torch.int64, device=dev)))
    out = torch.empty((1 << 20, dim), dtype=torch.float32, device=dev)
    found = [torch.empty(1 << 20, dtype=torch.uint8, device=dev) for _ in range(nsteps)]
    torch.cuda.synchronize()
    for j in range(args.warmup):
        tab.find(finds[j], values_out=out, found_out=found[j])
        tab.insert_or_assign(*ups[j])
    torch.cuda.synchronize()
    tab.profile_start()
    t1 = time.perf_counter()
    keys = 0
    for j in range(args.warmup, nsteps):
        tab.find(finds[j], values_out=out, found_out=found[j])
        tab.insert_or_assign(*ups[j])
        keys += finds[j].numel() + ups[j][0].numel()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    ks = tab.profile_stop()
    hits = sum(int(f.sum()) for f in found[args.warmup:]) / (args.steps * (1 << 20))
    find_ms = ks["find"][1] / ks["find"][0]
    up_ms = sum(ks[n][1] / ks[n][0] for n in ("upsert_probe", "upsert_owner"))
    up_keys = sum(u[0].numel() for u in ups[args.warmup:]) / args.steps
    key_side = 8 + 2 * 128 + 2 * 4 + hits * 8 + 1  # key, two digest lines, false positives, key, flag
    res = dict(
        workload=(f"tiered values: dual bucket, capacity 2^{args.capacity_log2}, dim {dim} rows in pinned host "
                  f"memory; per step find 2^20 Zipf(1.2) draws + insert_or_assign of 2^19 draws deduplicated"),
        combined_bkvs=round(keys / wall / 1e9, 4), find_bkvs=round((1 << 20) / find_ms / 1e6, 4),
        upsert_bkvs=round(up_keys / up_ms / 1e6, 4), hit_rate=round(hits, 4),
        find_kernel_ms=round(find_ms, 4), upsert_kernels_ms=round(up_ms, 4),
        find_key_side_hbm_GBps=round((1 << 20) * (key_side + hits * row) / (find_ms * 1e-3) / 1e9, 1),
        # rows delivered by find, repeats of hot keys counted each time
        find_row_GBps=round((1 << 20) * hits * row / (find_ms * 1e-3) / 1e9, 1),
        find_distinct_keys_per_batch=int(sum(torch.unique(f).numel() for f in finds[args.warmup:]) / args.steps),
        upsert_distinct_keys_per_batch=int(up_keys),
        upsert_row_write_GBps=round(up_keys * row / (ks["upsert_probe"][1] / ks["upsert_probe"][0] * 1e-3) / 1e9, 1),
        kernels={n: round(v[1] / v[0], 4) for n, v in ks.items()}, size=tab.size(), capacity=cap)
    log(f"tiered: {res}")
    tab.close()
    print(json.dumps({"tiered": res}), flush=True)


def assign_bytes_per_key(dim: int) -> float:
    """assign of a resident key: 8 key + 8 score in + 4D row in + 128 digest
    line + 4 false-positive keys + 8 key + 4D row write + 8 score write."""
    return 164 + 8 * dim


def triple_run(args) -> None:
    """The mixed reader / updater / inserter workload: one single-bucket table
    of 2^capacity_log2 slots (2^27) with dim --dim rows (64) filled to
    lambda = 1 with distinct uniform keys in 2^20-key batches (score = batch).
    Each step: find 2^20 keys (90 % resident, 10 % never inserted), assign
    2^19 distinct resident keys (new rows, score = step), insert_or_assign
    2^18 keys (2^17 resident, 2^17 new), on one stream. --warmup steps, then
    --steps timed steps with nothing but the calls queued (value = 1.75 * 2^20
    keys per step / wall time), then --steps more with kernel timing (rate of
    each call from its kernels' time). Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap, dim = 1 << args.capacity_log2, args.dim
    nf, na, nu = 1 << 20, 1 << 19, 1 << 18
    t0 = time.perf_counter()
    tab = H.HashTable(cap, dim)
    cursor, step, size = fill_table(tab, 1.0, cap, 1 << 20, dim, SEED, 800, dev)
    torch.cuda.synchronize()
    log(f"triple: filled to {size} with {cursor} keys in {time.perf_counter() - t0:.1f}s")
    # the last two fill batches: resident, and the highest-ranked keys, so no
    # insert of the measured steps evicts them
    pool = gen.unique_keys(SEED, 800, cursor - (2 << 20), 2 << 20, device=dev)
    n_hit = int(round(nf * 0.9))
    total = args.warmup + 2 * args.steps
    steps = []
    for j in range(total):
        pick = torch.argsort(gen.counter_words(SEED, 810, j * pool.numel(), pool.numel(), dev))
        fk = gen.shuffle(torch.cat([pool[pick[:n_hit]], gen.unique_keys(SEED, 811, j * nf, nf - n_hit, device=dev)]),
                         SEED, 820 + j)
        ak = pool[pick[n_hit:n_hit + na]]
        uk = gen.shuffle(torch.cat([pool[pick[-(nu // 2):]], gen.unique_keys(SEED, 812, j * nu, nu // 2, device=dev)]),
                         SEED, 900 + j)
        sc = step + 1 + j
        steps.append((fk, ak, torch.full((na,), sc, dtype=torch.int64, device=dev), uk,
                       torch.full((nu,), sc, dtype=torch.int64, device=dev)))
    a_rows = gen.values(pool[:na], 3000, dim, SEED)
    u_rows = gen.values(pool[:nu], 3001, dim, SEED)
    out = torch.empty((nf, dim), dtype=torch.float32, device=dev)
    found = [torch.empty(nf, dtype=torch.uint8, device=dev) for _ in range(total)]

    def run(first, count):
        for j in range(first, first + count):
            fk, ak, asc, uk, usc = steps[j]
            tab.find(fk, values_out=out, found_out=found[j])
            tab.assign(ak, a_rows, asc)
            tab.insert_or_assign(uk, u_rows, usc)

    torch.cuda.synchronize()
    run(0, args.warmup)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    tab.profile_start()
    run(args.warmup + args.steps, args.steps)
    ks = tab.profile_stop()
    hits = sum(int(f.sum()) for f in found[args.warmup:]) / (2 * args.steps * nf)
    avg = {n: v[1] / v[0] for n, v in ks.items()}
    call_ms = {"find": avg["find"], "assign": avg["assign"],
               "insert_or_assign": avg["upsert_probe"] + avg["upsert_owner"]}
    per_key = {"find": find_bytes_per_key(dim, hits), "assign": assign_bytes_per_key(dim),
               "upsert_probe": probe_bytes_per_key(dim, 0.5), "upsert_owner": owner_bytes_per_key(dim, 0.5, 1.0)}
    n_of = {"find": nf, "assign": na, "upsert_probe": nu, "upsert_owner": nu}
    kernels = {}
    for n in ("find", "assign", "upsert_probe", "upsert_owner"):
        gbs = n_of[n] * per_key[n] / (avg[n] * 1e-3) / 1e9
        kernels[n] = dict(avg_ms=round(avg[n], 5), bytes_per_launch=round(n_of[n] * per_key[n]),
                          achieved_GBps=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    res = dict(
        workload=(f"mixed reader/updater/inserter: single bucket, capacity 2^{args.capacity_log2}, dim {dim}, "
                  f"lambda 1.0; per step find 2^20 (90 % resident) + assign 2^19 resident + insert_or_assign "
                  f"2^18 (half new)"),
        combined_bkvs=round(1.75 * nf * args.steps / wall / 1e9, 4), ms_per_step=round(wall / args.steps * 1e3, 4),
        call_bkvs={n: round({"find": nf, "assign": na, "insert_or_assign": nu}[n] / ms / 1e6, 3)
                   for n, ms in call_ms.items()},
        kernel_step_ms=round(sum(call_ms.values()), 4), kernels=kernels, hit_rate=round(hits, 4),
        lambda_end=round(tab.size() / cap, 4), steps=args.steps, warmup=args.warmup)
    log(f"triple: {res}")
    tab.close()
    print(json.dumps({"triple": res}), flush=True)


def online_run(args) -> None:
    """Continuous online upsert at full capacity, single- against dual-bucket
    mode (the paper's §5.5, Table 11): a table of 2^capacity_log2 slots (2^27)
    with dim --dim rows (64) takes a stream of Zipf(1.05) draws over 2^30 ids
    (key = id), 2^20 draws per batch deduplicated, score = the key's
    cumulative frequency (LFU), until it is full, then 200 more batches.
    Before each batch's insert_or_assign, contains() looks up the batch's raw
    draws (the cache hit ratio) and its distinct keys (the fraction the upsert
    updates in place). find (rows copied out) is timed on a batch of
    raw draws once the table is half full and again at the end. Reported per
    mode: batches to fill,
    load factor at the first eviction (first batch that adds fewer keys than
    it has new ones), hit ratio and kernel-timed rates over the 200 batches,
    and top-N retention after them (N = capacity; ideal = the N highest
    (frequency, key) among all keys seen). Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap, dim, draws, n_ids, steady_batches = 1 << args.capacity_log2, args.dim, 1 << 20, 1 << 30, 200
    seed = 0x484B560000000003
    zipf = gen.Zipf(1.05, n_ids)
    out = {}
    for mode in args.online_modes.split(","):
        t0 = time.perf_counter()
        tab = H.HashTable(cap, dim, dual_bucket=mode == "dual")
        freq = torch.zeros(n_ids + 1, dtype=torch.int64, device=dev)
        rows_out = torch.empty((draws, dim), dtype=torch.float32, device=dev)
        found_out = torch.empty(draws, dtype=torch.uint8, device=dev)

        def find_ms(q):
            # find (rows copied out) on a batch of raw draws: kernel time
            tab.find(q, values_out=rows_out, found_out=found_out)
            tab.profile_start()
            for _ in range(3):
                tab.find(q, values_out=rows_out, found_out=found_out)
            ks = tab.profile_stop()
            return ks["find"][1] / ks["find"][0]

        b, size, first_evict, find_half = 0, 0, None, None
        while size < cap:
            r = zipf.draw(seed, 1, b * draws, draws, device=dev)
            uniq, cnt = torch.unique(r, return_counts=True)
            fresh = int((freq[uniq] == 0).sum())
            freq.index_add_(0, uniq, cnt)
            sc = freq[uniq]
            tab.insert_or_assign(uniq, gen.values(uniq, sc, dim, seed), sc)
            new_size = tab.size()
            if first_evict is None and new_size - size < fresh:
                first_evict = size / cap
            size = new_size
            b += 1
            if b % 200 == 0:
                log(f"online {mode}: {b} batches, lambda {size / cap:.4f}")
            if find_half is None and size >= cap // 2:
                find_half = (size / cap, find_ms(zipf.draw(seed, 1, b * draws, draws, device=dev)))
            if b > 4000:
                raise RuntimeError("table never reached full capacity")
        fill_batches = b
        # the steady-state batches, generated before the measured loop
        batches = []
        for j in range(steady_batches):
            r = zipf.draw(seed, 1, (b + j) * draws, draws, device=dev)
            uniq, cnt = torch.unique(r, return_counts=True)
            freq.index_add_(0, uniq, cnt)
            sc = freq[uniq]
            batches.append((r, uniq, gen.values(uniq, sc, dim, seed), sc))
        found = torch.empty(draws, dtype=torch.uint8, device=dev)
        found_u = torch.empty(draws, dtype=torch.uint8, device=dev)
        hits = torch.zeros(1, dtype=torch.int64, device=dev)
        resident_u = torch.zeros(1, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()
        log(f"online {mode}: full after {fill_batches} batches ({time.perf_counter() - t0:.1f}s), first eviction "
            f"at lambda {first_evict}")
        tab.profile_start()
        t1 = time.perf_counter()
        keys = 0
        for r, uniq, v, sc in batches:
            tab.contains(r, found_out=found)
            hits += found.sum()
            # the batch's distinct keys already resident (the upsert's update
            # fraction, for its algorithmic bytes)
            tab.contains(uniq, found_out=found_u[:uniq.numel()])
            resident_u += found_u[:uniq.numel()].sum()
            tab.insert_or_assign(uniq, v, sc)
            keys += uniq.numel()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t1
        ks = tab.profile_stop()
        up_ms = sum(ks[n][1] for n in ("upsert_probe", "upsert_owner")) / steady_batches
        look_ms = ks["contains"][1] / ks["contains"][0] if "contains" in ks else None
        find_full = find_ms(batches[-1][0])
        # top-N retention
        k, _, _, _ = tab.export_batch(with_values=False)
        seen = torch.nonzero(freq > 0).flatten()
        fs = freq[seen]
        o = torch.argsort(seen, descending=True)
        o = o[torch.argsort(fs[o], descending=True, stable=True)]
        mark = torch.zeros(n_ids + 1, dtype=torch.bool, device=dev)
        mark[seen[o[:cap]]] = True
        retention = int(mark[k].sum()) / cap
        res = dict(fill_batches=fill_batches, first_eviction_lambda=round(first_evict, 4) if first_evict else None,
                   hit_ratio=round(int(hits.item()) / (steady_batches * draws), 4),
                   resident_fraction_of_distinct=round(int(resident_u.item()) / max(keys, 1), 4),
                   top_n_retention=round(retention, 5), distinct_keys_per_batch=int(keys / steady_batches),
                   upsert_bkvs=round(keys / steady_batches / up_ms / 1e6, 3),
                   lookup_bkvs=round(draws / look_ms / 1e6, 3) if look_ms else None,
                   find_bkvs_at_half=round(draws / find_half[1] / 1e6, 3), half_lambda=round(find_half[0], 4),
                   find_bkvs_full=round(draws / find_full / 1e6, 3),
                   upsert_kernels_ms={n: round(ks[n][1] / ks[n][0], 4) for n in ("upsert_probe", "upsert_owner")},
                   combined_wall_bkvs=round((keys + steady_batches * draws) / wall / 1e9, 3),
                   size=int(k.numel()))
        log(f"online {mode}: {res}")
        out[mode] = res
        tab.close()
        del batches, freq, mark, seen, fs, o, k, rows_out, found_out
        torch.cuda.empty_cache()
    if "dual" in out and "single" in out:
        out["dual_over_single_upsert"] = round(out["dual"]["upsert_bkvs"] / out["single"]["upsert_bkvs"], 3)
    print(json.dumps({"online": out, "capacity": cap, "dim": dim, "zipf_alpha": 1.05, "ids": n_ids,
                      "draws_per_batch": draws, "steady_batches": steady_batches}), flush=True)


def graph_run(args) -> None:
    """Small, launch-bound batches (the tiny workload's shape: 2^16 slots, dim
    16, full, 16384-key batches): per step a find and an insert_or_assign of
    16384 keys, issued eagerly, then the same step captured once into a HIP
    graph and replayed. All calls on one stream (the table records no events)
    and the inserter workspace sized by the eager steps before capture. Rate =
    keys of the timed steps / wall time. Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap, dim, n = 1 << 16, 16, 16384
    s = torch.cuda.Stream()
    tab = H.HashTable(cap, dim)
    res = {}
    with torch.cuda.stream(s):
        for step in range(1, 9):
            k = gen.keys_in_range(SEED, step, n, 1, 1 << 40, device=dev)
            tab.insert_or_assign(k, gen.values(k, step, dim, SEED), torch.full((n,), step, dtype=torch.int64,
                                                                                 device=dev), stream=s)
        ek, _, _, _ = tab.export_batch(with_values=False, stream=s)
        half = ek[torch.randperm(ek.numel(), device=dev)[: n // 2]]
        qk = gen.shuffle(torch.cat([half, gen.unique_keys(SEED, 90, 0, n - half.numel(), device=dev)]), SEED, 91)
        uk = ek[torch.randperm(ek.numel(), device=dev)[:n]].contiguous()
        uv = gen.values(uk, 100, dim, SEED)
        us = torch.full((n,), 100, dtype=torch.int64, device=dev)
        out = torch.empty((n, dim), dtype=torch.float32, device=dev)
        found = torch.empty(n, dtype=torch.uint8, device=dev)

        def step_calls():
            tab.find(qk, values_out=out, found_out=found, stream=s)
            tab.insert_or_assign(uk, uv, us, stream=s)

        reps = max(args.steps, 20) * 10
        for _ in range(10):
            step_calls()
        s.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            step_calls()
        s.synchronize()
        eager = time.perf_counter() - t0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step_calls()
        for _ in range(10):
            g.replay()
        s.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        s.synchronize()
        graph = time.perf_counter() - t0
    res = dict(workload="2^16 slots, dim 16, full; per step find 16384 keys (half resident) + insert_or_assign of "
                        "16384 resident keys", steps=reps,
               eager_us_per_step=round(eager / reps * 1e6, 2), graph_us_per_step=round(graph / reps * 1e6, 2),
               eager_bkvs=round(2 * n * reps / eager / 1e9, 3), graph_bkvs=round(2 * n * reps / graph / 1e9, 3))
    log(f"graph: {res}")
    tab.close()
    print(json.dumps({"graph": res}), flush=True)


API_CONFIGS = (("A", 8, 27), ("B", 32, 27), ("C", 64, 26))  # (name, dim, log2 capacity), pure HBM


def api_sweep(args) -> None:
    """Every call on single-bucket tables of the paper's pure-HBM
    configurations (A: dim 8, 2^27 slots; B: dim 32, 2^27; C: dim 64, 2^26)
    at each load factor of --api-lambdas, 2^batch_log2-key batches: find (90 % resident), find*,
    contains, assign (resident keys), insert_or_assign, insert_and_evict and
    find_or_insert (90 % resident, 10 % new keys); 2 warm-up and 10 timed
    batches per call. Last, insert_or_assign of all-new keys, 2 warm-up and 3
    timed batches (lambda_end shows the drift). Rate = keys / kernel time per
    call (library events).
    Prints one JSON line."""
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    batch = 1 << args.batch_log2
    n_hit = int(round(batch * args.hit_frac))
    n_new = int(round(batch * args.new_frac))
    reps = 12
    out = {}
    for (name, dim, lg), lam in [(c, float(x)) for c in API_CONFIGS for x in args.api_lambdas.split(",")]:
        cap = 1 << lg
        tab = H.HashTable(cap, dim)
        cursor, step, size = fill_table(tab, lam, cap, batch, dim, SEED, 600, dev)
        pool = gen.unique_keys(SEED, 600, cursor - 2 * batch, 2 * batch, device=dev)
        finds, writes = [], []
        for j in range(reps):
            pick = torch.argsort(gen.counter_words(SEED, 610, j * pool.numel(), pool.numel(), dev))
            q = torch.cat([pool[pick[:n_hit]], gen.unique_keys(SEED, 611, j * batch, batch - n_hit, device=dev)])
            finds.append(gen.shuffle(q, SEED, 620 + j))
        for j in range(4 * reps):
            pick = torch.argsort(gen.counter_words(SEED, 612, j * pool.numel(), pool.numel(), dev))
            u = torch.cat([pool[pick[:batch - n_new]], gen.unique_keys(SEED, 613, j * batch, n_new, device=dev)])
            u = gen.shuffle(u, SEED, 700 + j)
            writes.append((u, gen.values(u, 2000 + j, dim, SEED),
                           torch.full((batch,), step + j, dtype=torch.int64, device=dev)))
        # all-new keys (the paper's insert_or_assign measurement: at lambda = 1
        # every insert evicts); few batches, so the load factor drifts little
        new_reps = 5
        fresh = [gen.unique_keys(SEED, 614, j * batch, batch, device=dev) for j in range(new_reps)]
        fresh = [(u, gen.values(u, 3000 + j, dim, SEED), torch.full((batch,), step + 4 * reps + j, dtype=torch.int64,
                                                                     device=dev)) for j, u in enumerate(fresh)]
        vals = torch.empty((batch, dim), dtype=torch.float32, device=dev)
        found = torch.empty(batch, dtype=torch.uint8, device=dev)
        ptrs = torch.empty(batch, dtype=torch.int64, device=dev)
        ev = (torch.empty(batch, dtype=torch.int64, device=dev), torch.empty((batch, dim), device=dev),
              torch.empty(batch, dtype=torch.int64, device=dev), torch.zeros(1, dtype=torch.int64, device=dev))
        calls = {
            "find": lambda j: tab.find(finds[j], values_out=vals, found_out=found),
            "find_ptr": lambda j: tab.find_ptr(finds[j], ptrs_out=ptrs, found_out=found),
            "contains": lambda j: tab.contains(finds[j], found_out=found),
            "assign": lambda j: tab.assign(finds[j][:n_hit], writes[j][1][:n_hit], writes[j][2][:n_hit]),
            "insert_or_assign": lambda j: tab.insert_or_assign(*writes[j]),
            "insert_and_evict": lambda j: tab.insert_and_evict(*writes[reps + j], out=ev),
            "find_or_insert": lambda j: tab.find_or_insert(writes[2 * reps + j][0], writes[2 * reps + j][1],
                                                           writes[2 * reps + j][2], found_out=found),
            "insert_or_assign_new_keys": lambda j: tab.insert_or_assign(*fresh[j]),
        }
        res = {}
        for api, call in calls.items():
            n_calls = new_reps if api == "insert_or_assign_new_keys" else reps
            for j in range(2):
                call(j)
            torch.cuda.synchronize()
            tab.profile_start()
            for j in range(2, n_calls):
                call(j)
            ks = tab.profile_stop()
            per_call = sum(v[1] for v in ks.values()) / (n_calls - 2)
            keys = n_hit if api == "assign" else batch
            res[api] = round(keys / per_call / 1e6, 3)
        res["lambda_end"] = round(tab.size() / cap, 4)
        out[f"{name}: dim {dim}, 2^{lg} slots, lambda {lam}"] = res
        log(f"config {name} lambda {lam}: {res}")
        tab.close()
        del finds, writes, fresh
        torch.cuda.empty_cache()
    print(json.dumps({"api_sweep_bkvs": out, "batch": batch}), flush=True)


MIXES = {
    "1U": "U", "2U": "UU", "5U": "UUUUU", "10U": "UUUUUUUUUU",
    "4F/5U/1I": "FFFFUUUUUI", "4F/2U/4I": "FFFFUUIIII", "8F/1U/1I": "FFFFFFFFUI",
}


def mixed_sweep(args) -> None:
    """Concurrency ablation (the paper's §5.4): host threads share one table,
    each issuing back-to-back batches of one role (F find, U assign,
    I insert_or_assign) on its own stream through the native multi-threaded
    driver; the table orders the calls either by the three groups (readers
    with readers, updaters with updaters) or, with HKV_FLAG_RW_LOCK, as a
    reader/writer lock (only readers overlap). Single-bucket table of
    2^capacity_log2 slots at lambda 0.75, dim from --dim (16 in the paper's
    runs), batches of 2^16 keys: finds and assigns of resident keys, inserts
    of half resident, half new keys; --mixed-batches per thread, median of
    three timed runs. value = keys of all threads / wall time. Prints one
    JSON line."""
    import ctypes

    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen
    from hash_table_cache_amd import build as hb

    lib = ctypes.CDLL(str(hb.MIXED_LIB_PATH))
    P = ctypes.c_void_p
    lib.hkv_mixed_run.argtypes = [P, ctypes.c_uint32, P, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32,
                                  P, P, P, P, P, ctypes.POINTER(ctypes.c_double)]
    lib.hkv_mixed_run.restype = ctypes.c_int32
    dev = torch.device("cuda", 0)
    cap, dim = 1 << args.capacity_log2, args.dim
    batch, pool, nb = 1 << 16, 4, args.mixed_batches
    out = {}
    for mix in args.mixed.split(","):
        roles = MIXES[mix]
        res = {}
        for mode in ("triple_group", "rw_lock"):
            flags = H.HKV_FLAG_RW_LOCK if mode == "rw_lock" else 0
            tab = H.HashTable(cap, dim, flags=flags)
            fill_table(tab, 0.75, cap, 1 << 20, dim, SEED, 300, dev)
            k_all, _, _, _ = tab.export_batch(with_values=False)
            bufs, ptrs = [], {n: [] for n in ("keys", "values", "scores", "out", "found")}
            for j, r in enumerate(roles):
                pick = torch.argsort(gen.counter_words(SEED, 310 + j, 0, k_all.numel(), dev))[:pool * batch]
                k = k_all[pick]
                if r == "I":
                    k = k.view(pool, batch)
                    fresh = gen.unique_keys(SEED, 330 + j, 0, pool * batch // 2, device=dev).view(pool, -1)
                    k = torch.cat([k[:, :batch // 2], fresh], 1).reshape(-1).contiguous()
                v = gen.values(k, 900 + j, dim, SEED)
                sc = torch.full((pool * batch,), 1 << 20, dtype=torch.int64, device=dev)
                o = torch.empty((batch, dim), dtype=torch.float32, device=dev)
                f = torch.empty(batch, dtype=torch.uint8, device=dev)
                bufs.append((k, v, sc, o, f))
                for n, t in zip(("keys", "values", "scores", "out", "found"), (k, v, sc, o, f)):
                    ptrs[n].append(t.data_ptr())
            torch.cuda.synchronize()
            arr = {n: (ctypes.c_void_p * len(roles))(*v) for n, v in ptrs.items()}
            role_ids = (ctypes.c_int32 * len(roles))(*["FUI".index(r) for r in roles])
            secs = ctypes.c_double(0)
            # one short untimed pass, then three timed ones (median)
            times = []
            for timed_batches in (4, nb, nb, nb):
                st = lib.hkv_mixed_run(tab.handle, len(roles), role_ids, timed_batches, batch, pool,
                                       arr["keys"], arr["values"], arr["scores"], arr["out"], arr["found"],
                                       ctypes.byref(secs))
                if st != 0:
                    raise RuntimeError(f"hkv_mixed_run status {st}")
                times.append(secs.value)
            t = sorted(times[1:])[1]
            res[mode] = dict(seconds=round(t, 5), bkvs=round(len(roles) * nb * batch / t / 1e9, 3))
            del bufs
            tab.close()
            torch.cuda.empty_cache()
        res["ratio"] = round(res["triple_group"]["bkvs"] / res["rw_lock"]["bkvs"], 3)
        log(f"mix {mix}: {res}")
        out[mix] = res
    print(json.dumps({"mixed": out, "capacity": cap, "dim": dim, "batch": batch, "batches_per_thread": nb,
                      "lambda": 0.75}), flush=True)


def fill_table(tab, lam, cap, batch, dim, seed, stream_id, device):
    """Upserts fresh distinct keys (score = batch counter) until size >= lam*cap.
    Returns (next counter of the key stream, next score)."""
    import torch

    import hkv_inputs as gen

    target = int(round(lam * cap))
    cursor, step, size = 0, 1, 0
    while size < target:
        n = batch if lam >= 1.0 else min(batch, target - size)
        keys = gen.unique_keys(seed, stream_id, cursor, n, device=device)
        vals = gen.values(keys, step, dim, seed)
        sc = torch.full((n,), step, dtype=torch.int64, device=device)
        tab.insert_or_assign(keys, vals, sc)
        cursor += n
        step += 1
        size = tab.size()
    return cursor, step, size


def run_gpu(args):
    import numpy as np
    import torch

    import hash_table_cache_amd as H
    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    cap = 1 << args.capacity_log2
    batch = 1 << args.batch_log2
    dim = args.dim
    lams = [float(x) for x in args.lambdas.split(",")]
    # warm-up, the timed steps (nothing but the calls), then as many again
    # with kernel timing on (per-kernel times, roofline, per-lambda rates)
    total_steps = args.warmup + 2 * args.steps
    tables = []
    cpu_sample = None
    for li, lam in enumerate(lams):
        t0 = time.perf_counter()
        tab = H.HashTable(cap, dim, device=0, unique_keys=args.unique_keys)
        cursor, step, size = fill_table(tab, lam, cap, batch, dim, SEED, 1 + li, dev)
        torch.cuda.synchronize()
        log(f"lambda={lam}: filled to size {size} ({size / cap:.4f}) with {cursor} keys "
            f"in {time.perf_counter() - t0:.1f}s")
        # Inputs of every step, generated now (outside the timed region).
        # --hit-pool resident: each step's resident keys are sampled uniformly
        # from the table's resident set as it is at that step: an untimed dry
        # run on this table applies every step's upsert and exports the
        # resident set before each step; a fresh table filled the same way
        # (the same contents, single-bucket mode) then runs the steps. So the
        # find batches hold exactly the hit fraction at every load factor.
        # --hit-pool recent: from the 2^(batch+1) most recently inserted keys.
        n_hit = int(round(batch * args.hit_frac))
        n_new = int(round(batch * args.new_frac))
        finds, ups = [], []
        vals_pool = None
        for s in range(total_steps):
            if args.hit_pool == "resident":
                pool = tab.export_batch(with_values=False)[0]
            else:
                recent = min(cursor, 2 * batch)
                pool = gen.unique_keys(SEED, 1 + li, cursor - recent, recent, device=dev)
            n_pool = pool.numel()
            if vals_pool is None:
                vals_pool = [gen.values(pool[:batch], 1000 + j, dim, SEED) for j in range(2)]
            pick = torch.argsort(gen.counter_words(SEED, 100 + li, s * n_pool, n_pool, dev))
            hits = pool[pick[:n_hit]]
            miss = gen.unique_keys(SEED, 40 + li, s * batch, batch - n_hit, device=dev)
            fk = gen.shuffle(torch.cat([hits, miss]), SEED, 200 + li * 1000 + s)
            res = (pool[pick[n_hit:n_hit + (batch - n_new)]] if batch - n_new <= n_pool - n_hit
                   else pool[pick[:batch - n_new]])
            del pick, pool
            new = gen.unique_keys(SEED, 60 + li, s * batch, n_new, device=dev)
            uk = gen.shuffle(torch.cat([res, new]), SEED, 300 + li * 1000 + s)
            sc = torch.full((batch,), step + s, dtype=torch.int64, device=dev)
            finds.append(fk)
            ups.append((uk, sc))
            if args.hit_pool == "resident" and not args.find_only:
                tab.insert_or_assign(uk, vals_pool[s % 2], sc)
        if args.hit_pool == "resident" and not args.find_only:
            tab.close()
            torch.cuda.synchronize()
            tab = H.HashTable(cap, dim, device=0, unique_keys=args.unique_keys)
            fill_table(tab, lam, cap, batch, dim, SEED, 1 + li, dev)
        if li == 0 and not args.no_cpu_baseline and not args.find_only:
            # the batches the CPU oracle replays: the warm-up steps and the
            # first timed steps of this table, copied to the host
            cpu_steps = args.warmup + min(args.steps, args.cpu_steps)
            cpu_sample = dict(lam=lam, li=li, warmup=args.warmup, batches=[
                (finds[s].cpu().numpy().view(np.uint64), ups[s][0].cpu().numpy().view(np.uint64),
                 ups[s][1].cpu().numpy().view(np.uint64)) for s in range(cpu_steps)])
        out = torch.empty((batch, dim), dtype=torch.float32, device=dev)
        found = [torch.empty(batch, dtype=torch.uint8, device=dev) for _ in range(total_steps)]
        tables.append(dict(lam=lam, tab=tab, finds=finds, ups=ups, vals=vals_pool, out=out, found=found,
                           lam_start=size / cap))
    torch.cuda.synchronize()

    total_keys = 0

    def table_step(T, s, timed):
        # warm-up steps run exactly the same calls as timed ones; nothing but
        # the calls is queued (kernel times come from the dispatches' events)
        nonlocal total_keys
        T["tab"].find(T["finds"][s], values_out=T["out"], found_out=T["found"][s])
        if not args.find_only:
            uk, sc = T["ups"][s]
            T["tab"].insert_or_assign(uk, T["vals"][s % 2], sc)
        if timed:
            total_keys += batch * (1 if args.find_only else 2)

    def run_steps(first, count, timed):
        # A step is one find and one insert_or_assign on every table. By
        # default the steps of a phase are grouped by table — every step on
        # the first load factor's table, then the next — as the paper measures
        # each load factor on a table of its own; --interleave-tables runs
        # step by step across the tables instead (their digest arrays then
        # compete for the caches between consecutive batches).
        if args.interleave_tables:
            for s in range(first, first + count):
                for T in tables:
                    table_step(T, s, timed)
        else:
            for T in tables:
                for s in range(first, first + count):
                    table_step(T, s, timed)

    run_steps(0, args.warmup, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.warmup, args.steps, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for T in tables:
        T["size0"] = T["tab"].size()
        T["tab"].profile_start()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run_steps(args.warmup + args.steps, args.steps, False)
    torch.cuda.synchronize()
    wall_timed_kernels = time.perf_counter() - t1
    kstats = {}
    for T in tables:
        T["kernels"] = T["tab"].profile_stop()
        for name, (cnt, tot, *_) in T["kernels"].items():
            a = kstats.setdefault(name, [0, 0.0])
            a[0] += cnt
            a[1] += tot

    hit = {}
    for T in tables:
        hits = sum(int(f.sum().item()) for f in T["found"][args.warmup:])
        hit[T["lam"]] = hits / (batch * 2 * args.steps)
        T["lam_end"] = T["tab"].size() / cap
    h_avg = sum(hit.values()) / len(hit)
    # per-lambda call times: the table's kernel times per call (find: one
    # kernel; insert_or_assign: probe + owner)
    detail = {}
    for T in tables:
        ks = T["kernels"]
        fm = ks["find"][1] / ks["find"][0]
        e = dict(find_ms=round(fm, 5), find_bkvs=round(batch / fm / 1e6, 3), hit_rate=round(hit[T["lam"]], 4),
                 find_cv=launch_cv(ks["find"]))
        if not args.find_only:
            um = sum(ks[k][1] / ks[k][0] for k in ("upsert_probe", "upsert_owner"))
            e.update(upsert_ms=round(um, 5), upsert_bkvs=round(batch / um / 1e6, 3),
                     upsert_probe_cv=launch_cv(ks["upsert_probe"]), upsert_owner_cv=launch_cv(ks["upsert_owner"]))
        e.update(lambda_start=round(T["lam_start"], 4), lambda_end=round(T["lam_end"], 4))
        detail[str(T["lam"])] = e
    fb = [v["find_bkvs"] for v in detail.values()]
    find_var = (max(fb) - min(fb)) / max(fb)
    # algorithmic bytes per launch of each kernel, averaged over the tables
    f_res = 1.0 - args.new_frac
    n_new = int(round(batch * args.new_frac)) * args.steps
    bytes_per_launch = {"find": 0.0, "upsert_probe": 0.0, "upsert_owner": 0.0}
    for T in tables:
        inserted = T["tab"].size() - T["size0"]
        e = max(0.0, 1.0 - inserted / n_new) if n_new else 0.0
        T["evict_frac"] = e
        bytes_per_launch["find"] += batch * find_bytes_per_key(dim, hit[T["lam"]]) / len(tables)
        bytes_per_launch["upsert_probe"] += batch * probe_bytes_per_key(dim, f_res) / len(tables)
        bytes_per_launch["upsert_owner"] += batch * owner_bytes_per_key(dim, f_res, e) / len(tables)
        detail[str(T["lam"])]["evicting_new_frac"] = round(e, 4)
        detail[str(T["lam"])]["kernel_avg_ms"] = {k: round(v[1] / v[0], 5) for k, v in T["kernels"].items()}
    kernels = {}
    for name, (cnt, tot) in kstats.items():
        k = dict(launches=cnt, total_ms=round(tot, 3), avg_ms=round(tot / cnt, 5))
        if name in bytes_per_launch:
            gbs = bytes_per_launch[name] / (tot / cnt * 1e-3) / 1e9
            k.update(bytes_per_launch=round(bytes_per_launch[name]), achieved_GBps=round(gbs, 1),
                     frac=round(gbs / HBM_PEAK_GBS, 4))
        kernels[name] = k
    dominant = max(kernels, key=lambda n: kernels[n]["total_ms"])
    # Eviction-heavy phase (reported in detail only): all-new keys into the
    # full table, every key lands in a full bucket (evict or reject).
    insert_new = None
    full = [T for T in tables if T["lam"] >= 1.0]
    if full and args.insert_steps > 0:
        T = full[0]
        tab = T["tab"]
        batches = []
        for j in range(args.insert_steps + 1):
            k = gen.unique_keys(SEED, 90, j * batch, batch, device=dev)
            batches.append((k, gen.values(k, 5000 + j, dim, SEED),
                            torch.full((batch,), 10_000 + j, dtype=torch.int64, device=dev)))
        tab.insert_or_assign(*batches[0])
        torch.cuda.synchronize()
        tab.profile_start()
        t1 = time.perf_counter()
        for k, v, sc in batches[1:]:
            tab.insert_or_assign(k, v, sc)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        ks = tab.profile_stop()
        insert_new = dict(batches=args.insert_steps, bkvs=round(args.insert_steps * batch / dt / 1e9, 3),
                          kernel_avg_ms={n: round(v[1] / v[0], 5) for n, v in ks.items()},
                          lambda_end=round(tab.size() / cap, 4))
    extra_ops = run_extra_ops(args, tables, batch, dim, hit) if args.extra_ops else None
    for T in tables:
        T["tab"].close()
    busy = sum(v[1] for v in kstats.values())
    # algorithmic bytes of one whole step (every kernel on every table)
    step_bytes = sum(bytes_per_launch[name] for name in kstats if name in bytes_per_launch) * len(tables)
    return dict(wall=wall, total_keys=total_keys, detail=detail, find_var=find_var, kernels=kernels,
                dominant=dominant, h=h_avg, gpu_busy_frac=busy / (wall_timed_kernels * 1e3),
                wall_timed_kernels=wall_timed_kernels, insert_new=insert_new, extra_ops=extra_ops,
                step_bytes=step_bytes, cpu_sample=cpu_sample)


def run_extra_ops(args, tables, batch, dim, hit):
    """The other calls of the paper's §4.1 on the same tables, after the timed
    region (reported in detail only): find* and contains on the step's find
    batches, and find with the stored scores returned (kernel time; 16 more
    bytes per hit: score read and written); insert_and_evict, then
    find_or_insert, on fresh batches of the
    upsert mix (90 % resident, 10 % new keys). Per call: median of HIP-event
    times around the call; per kernel: the library's event times."""
    import torch

    import hkv_inputs as gen

    dev = torch.device("cuda", 0)
    reps = min(args.steps, 10)
    out = {}
    for li, T in enumerate(tables):
        tab = T["tab"]
        lam = T["lam"]
        r = {}
        ptrs = torch.empty(batch, dtype=torch.int64, device=dev)
        found = torch.empty(batch, dtype=torch.uint8, device=dev)
        for name in ("find_ptr", "contains"):
            ms = []
            for s in range(reps + 2):
                if s == 2:  # two warm-up calls, untimed in both measures
                    torch.cuda.synchronize()  # no queued work ahead of the first timed launch
                    tab.profile_start()
                if s == reps // 2 + 2:  # kernel times above, call times below
                    ks = tab.profile_stop()
                q = T["finds"][s % len(T["finds"])]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if name == "find_ptr":
                    tab.find_ptr(q, ptrs_out=ptrs, found_out=found)
                else:
                    tab.contains(q, found_out=found)
                e1.record()
                ms.append((e0, e1))
            torch.cuda.synchronize()
            timed = ms[reps // 2 + 2:]
            t = sorted(a.elapsed_time(b) for a, b in timed)[len(timed) // 2]
            kn = ks[name]
            kavg = kn[1] / kn[0]
            byts = batch * locate_bytes_per_key(hit[lam], name == "find_ptr")
            r[name] = dict(call_ms_median=round(t, 5), bkvs=round(batch / t / 1e6, 3), kernel_avg_ms=round(kavg, 5),
                           achieved_GBps=round(byts / (kavg * 1e-3) / 1e9, 1),
                           frac=round(byts / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        # find with the stored scores returned (the metric's one extra run)
        scs = torch.empty(batch, dtype=torch.int64, device=dev)
        for s in range(reps + 2):
            if s == 2:
                torch.cuda.synchronize()
                tab.profile_start()
            tab.find(T["finds"][s % len(T["finds"])], values_out=T["out"], found_out=found, scores_out=scs)
        ks = tab.profile_stop()
        kavg = ks["find"][1] / ks["find"][0]
        byts = batch * (find_bytes_per_key(dim, hit[lam]) + 16 * hit[lam])
        r["find_with_scores"] = dict(kernel_avg_ms=round(kavg, 5), bkvs=round(batch / kavg / 1e6, 3),
                                     achieved_GBps=round(byts / (kavg * 1e-3) / 1e9, 1),
                                     frac=round(byts / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        # export of the whole table with rows (checkpointing, §4.1): kernel time
        tab.export_batch(with_values=True)
        torch.cuda.empty_cache()
        tab.profile_start()
        ek, ev_, es_, ep_ = tab.export_batch(with_values=True)
        ks = tab.profile_stop()
        ex_ms = ks["export"][1] / ks["export"][0]
        ex_bytes = ek.numel() * (8 + 8 + 4 * dim) * 2 + tab.capacity // 128 * 4  # read + write, occupancy words
        r["export_with_rows"] = dict(entries=int(ek.numel()), kernel_ms=round(ex_ms, 4),
                                     bkvs=round(ek.numel() / ex_ms / 1e6, 3),
                                     GBps=round(ex_bytes / (ex_ms * 1e-3) / 1e9, 1))
        del ek, ev_, es_, ep_
        torch.cuda.empty_cache()
        # write calls on fresh batches of the upsert mix
        n_new = int(round(batch * args.new_frac))
        k_all, _, _, _ = tab.export_batch(with_values=False)
        evk = torch.empty(batch, dtype=torch.int64, device=dev)
        evv = torch.empty((batch, dim), dtype=torch.float32, device=dev)
        evs = torch.empty(batch, dtype=torch.int64, device=dev)
        score0 = 1 << 30
        batches = []
        for j in range(2 * (reps + 2)):
            pick = torch.argsort(gen.counter_words(SEED, 500 + li, j * k_all.numel(), k_all.numel(), dev))
            res = k_all[pick[:batch - n_new]]
            new = gen.unique_keys(SEED, 520 + li, j * batch, n_new, device=dev)
            uk = gen.shuffle(torch.cat([res, new]), SEED, 540 + li * 1000 + j)
            batches.append((uk, gen.values(uk, 7000 + j, dim),
                            torch.full((batch,), score0 + j, dtype=torch.int64, device=dev)))
        torch.cuda.synchronize()
        # Each call is timed with events around it in one pass, and its kernels
        # with the library's per-kernel events in a second pass on fresh
        # batches (per-kernel events add host work per launch, which would
        # leave the GPU waiting inside the timed calls). Each
        # insert_and_evict call writes its own hand-back count. The per-kernel
        # events start one call after the synchronize: a kernel's event pair
        # opens when the stream reaches its start marker, and on an idle GPU
        # (just synchronized) that can precede the kernel's own dispatch by a
        # host submission gap (up to ~1 ms seen for insert_and_evict's probe,
        # whose dispatches all take 0.15-0.2 ms in rocprofv3's kernel trace).
        cnts = torch.zeros(reps + 2, dtype=torch.int64, device=dev)
        for name, part in (("insert_and_evict", batches[:reps + 2]), ("find_or_insert", batches[reps + 2:])):
            ms = []
            for j, (uk, uv, usc) in enumerate(part):
                if j == 2:  # the first two calls (workspace growth) are warm-up in both measures
                    torch.cuda.synchronize()
                if j == 3:
                    tab.profile_start()
                if j == reps // 2 + 2:  # the rest of the calls: call times only
                    ks = tab.profile_stop()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if name == "insert_and_evict":
                    tab.insert_and_evict(uk, uv, usc, out=(evk, evv, evs, cnts[j:j + 1]))
                else:
                    tab.find_or_insert(uk, uv, usc, found_out=found)
                e1.record()
                ms.append((e0, e1))
            torch.cuda.synchronize()
            timed = ms[reps // 2 + 2:]
            t = sorted(a.elapsed_time(b) for a, b in timed)[len(timed) // 2]
            # per kernel: median, average, fastest and slowest launch (a
            # launch whose start event was taken before its dispatch moves
            # the average and the maximum, not the median)
            r[name] = dict(call_ms_median=round(t, 5), bkvs=round(batch / t / 1e6, 3),
                           kernel_median_ms={k: round(v[5], 5) for k, v in ks.items()},
                           kernel_avg_ms={k: round(v[1] / v[0], 5) for k, v in ks.items()},
                           kernel_min_max_ms={k: [round(v[3], 5), round(v[2], 5)] for k, v in ks.items()})
            if name == "insert_and_evict":
                r[name]["handed_back_per_call"] = round(float(cnts[2:].double().mean().item()), 1)
        out[str(lam)] = r
        log(f"lambda={lam}: other calls {r}")
    return out


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def run_cpu_baseline(args, sample):
    """The CPU oracle, single-threaded and pinned to one core, on the
    benchmark's own batches: the oracle builds the first load factor's table
    at the benchmark's capacity from the same fill batches (rows kept as
    8-byte version tags, the oracle's tag mode), replays the warm-up steps
    untimed, then applies the first timed steps' find and insert_or_assign
    batches (copied from the GPU run), each timed on its own. value = median
    over those steps of (keys of the step's two batches) / (their time)."""
    import numpy as np

    import hkv_inputs as gen
    import oracle

    cap = 1 << args.capacity_log2
    batch = 1 << args.batch_log2
    lam, li = sample["lam"], sample["li"]
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    try:
        t_all = time.perf_counter()
        o = oracle.OracleTable(cap, args.dim, tag_mode=True)
        target = int(round(lam * cap))
        cursor, step, size = 0, 1, 0
        while size < target:  # the same fill batches as fill_table()
            n = batch if lam >= 1.0 else min(batch, target - size)
            k = gen.unique_keys(SEED, 1 + li, cursor, n).numpy().view(np.uint64)
            tags = np.full(n, step, np.uint64)
            o.insert_or_assign(k, tags, tags=tags)
            cursor += n
            step += 1
            size = o.size()
        t_fill = time.perf_counter() - t_all
        find_s, up_s = [], []
        for s, (fk, uk, sc) in enumerate(sample["batches"]):
            t0 = time.perf_counter()
            o.find(fk)
            t1 = time.perf_counter()
            o.insert_or_assign(uk, sc, tags=sc)
            t2 = time.perf_counter()
            if s >= sample["warmup"]:
                find_s.append(t1 - t0)
                up_s.append(t2 - t1)
        o.close()
    finally:
        os.sched_setaffinity(0, set(allowed))
    per_step = [2 * batch / (a + b) / 1e9 for a, b in zip(find_s, up_s)]
    return dict(value=statistics.median(per_step), secs=sum(find_s) + sum(up_s), total=time.perf_counter() - t_all,
                fill_s=t_fill, steps=len(per_step), lam=lam, cap=cap, batch=batch, core=core,
                find_bkvs=statistics.median(batch / t / 1e9 for t in find_s),
                upsert_bkvs=statistics.median(batch / t / 1e9 for t in up_s),
                cpu_model=cpu_model(), nproc=os.cpu_count(), allowed=len(allowed))


def cold_runs(args):
    """The lambda sweep K times, each in a child process of its own (a cold
    start: new process, new tables, filled from empty), then the median over
    the runs of every per-lambda rate and of the combined value. This process
    never touches the GPU itself."""
    cmd = [sys.executable, os.path.abspath(__file__), "--no-cpu-baseline", "--no-extra-ops", "--insert-steps", "0",
           "--dim", str(args.dim), "--capacity-log2", str(args.capacity_log2), "--batch-log2", str(args.batch_log2),
           "--lambdas", args.lambdas, "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--hit-frac", str(args.hit_frac), "--new-frac", str(args.new_frac), "--hit-pool", args.hit_pool]
    runs = []
    for r in range(args.cold_runs):
        log(f"cold run {r + 1} of {args.cold_runs}")
        out = subprocess.run(cmd, capture_output=True, text=True)
        if out.returncode != 0:
            log(out.stderr[-2000:])
            raise SystemExit(f"cold run {r + 1} failed with status {out.returncode}")
        runs.append(json.loads(out.stdout.strip().splitlines()[-1]))
    med = lambda xs: float(statistics.median(xs))
    per = {}
    for lam in runs[0]["detail"]["per_lambda"]:
        rows = [r["detail"]["per_lambda"][lam] for r in runs]
        per[lam] = {k: round(med([x[k] for x in rows]), 3) for k in ("find_bkvs", "upsert_bkvs")}
        per[lam]["find_bkvs_runs"] = [x["find_bkvs"] for x in rows]
    fb = [v["find_bkvs"] for v in per.values()]
    print(json.dumps({"cold_runs": args.cold_runs, "dim": args.dim, "capacity_log2": args.capacity_log2,
                      "combined_bkvs_median": round(med([r["value"] for r in runs]), 4),
                      "combined_bkvs_runs": [r["value"] for r in runs],
                      "per_lambda_median": per,
                      "find_lambda_variation": round((max(fb) - min(fb)) / max(fb), 4)}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the table is a single-GPU "
              "structure and sharding it across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.capacity_sweep:
        capacity_sweep(args)
        return
    if args.hybrid:
        hybrid_sweep(args)
        return
    if args.mixed:
        mixed_sweep(args)
        return
    if args.tiered:
        tiered_run(args)
        return
    if args.api_sweep:
        api_sweep(args)
        return
    if args.triple:
        triple_run(args)
        return
    if args.online:
        online_run(args)
        return
    if args.graph:
        graph_run(args)
        return
    if args.cold_runs:
        cold_runs(args)
        return
    g = run_gpu(args)
    g["copy_GBps"] = copy_bandwidth()
    log(f"device copy bandwidth {g['copy_GBps']:.1f} GB/s")
    g["pattern"] = (pattern_ceiling(args.dim) if args.dim in (32, 64, 128) and args.capacity_log2 == 26
                    else None)
    cpu = None
    if not args.no_cpu_baseline and g.get("cpu_sample"):
        log("running the CPU oracle baseline")
        cpu = run_cpu_baseline(args, g["cpu_sample"])
        log(f"cpu baseline: {cpu['value'] * 1e3:.3f} M-KV/s over {cpu['secs']:.1f}s timed, {cpu['total']:.1f}s total "
            f"({cpu['fill_s']:.1f}s to fill)")
    value = g["total_keys"] / g["wall"] / 1e9
    n_lams = len(args.lambdas.split(","))
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "B-KV/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {
            "workload": (f"lambda sweep, single-bucket, capacity 2^{args.capacity_log2}, dim {args.dim} fp32 rows, "
                         f"uniform distinct u64 keys, per step per lambda: find 2^{args.batch_log2} "
                         f"({int(args.hit_frac * 100)}% resident)"
                         + ("" if args.find_only else
                            f" + insert_or_assign 2^{args.batch_log2} ({int(round((1 - args.new_frac) * 100))}% resident, "
                            f"{int(round(args.new_frac * 100))}% new), scores = step counter")
                         + ("; resident keys sampled uniformly from the whole resident set"
                            if args.hit_pool == "resident" else
                            "; resident keys sampled from the 2^(batch+1) most recently inserted")),
            "capacity": 1 << args.capacity_log2,
            "dim": args.dim,
            "batch": 1 << args.batch_log2,
            "lambdas": [float(x) for x in args.lambdas.split(",")],
            "tables": n_lams,
            "bucket_mode": "single",
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": g["dominant"],
            "bound": "hbm",
            "achieved": g["kernels"][g["dominant"]]["achieved_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": g["kernels"][g["dominant"]]["frac"],
            "traffic": profiled_traffic(g["dominant"], args.dim, args.capacity_log2),
            "bytes_per_launch": g["kernels"][g["dominant"]]["bytes_per_launch"],
            "avg_launch_ms": g["kernels"][g["dominant"]]["avg_ms"],
        },
        "cpu_baseline": None if cpu is None else {
            "value": round(cpu["value"], 6),
            "unit": "B-KV/s",
            "cores": 1,
            "kind": "oracle",
            "sample": (f"the oracle single-threaded, pinned to core {cpu['core']} of {cpu['allowed']} "
                       f"({cpu['cpu_model']}, nproc {cpu['nproc']}), on the benchmark's own lambda {cpu['lam']} "
                       f"table: capacity 2^{args.capacity_log2}, rows as 8-byte version tags, filled from the same "
                       f"batches ({cpu['fill_s']:.0f}s), the {args.warmup} warm-up steps replayed, then the first "
                       f"{cpu['steps']} timed steps' 2^{args.batch_log2}-key find and insert_or_assign batches "
                       f"copied from the GPU run, median over steps; {cpu['secs']:.1f}s timed"),
            "cpu_model": cpu["cpu_model"],
            "nproc": cpu["nproc"],
            "capacity": cpu["cap"],
            "find_bkvs_median": round(cpu["find_bkvs"], 6),
            "upsert_bkvs_median": round(cpu["upsert_bkvs"], 6),
        },
        "detail": {
            "kernels": g["kernels"],
            "kernel_timing_pass_ms_per_step": round(g["wall_timed_kernels"] / args.steps * 1e3, 4),
            "gpu_busy_frac_kernel_timing_pass": round(g["gpu_busy_frac"], 4),
            "per_lambda": g["detail"],
            "find_lambda_variation": round(g["find_var"], 4),
            "insert_all_new_at_lambda_1": g["insert_new"],
            "other_calls_per_lambda": g["extra_ops"],
            "copy_GBps": round(g["copy_GBps"], 1),
            "find_pattern_ceiling": g["pattern"],
            "find_frac_of_pattern_ceiling": (round(g["pattern"]["dependent_chain"]["us_per_2p20_keys"] * 1e-3
                                                  * batch_size(args) / (1 << 20) / g["kernels"]["find"]["avg_ms"], 4)
                                             if g["pattern"] else None),
            "upsert_probe_frac_of_pattern_ceiling": (
                round(g["pattern"]["upsert_probe_dependent_chain"]["us_per_2p20_keys"] * 1e-3 * batch_size(args)
                      / (1 << 20) / g["kernels"]["upsert_probe"]["avg_ms"], 4)
                if g["pattern"] and "upsert_probe" in g["kernels"] else None),
            "dominant_frac_of_copy": round(g["kernels"][g["dominant"]]["achieved_GBps"] / g["copy_GBps"], 4),
            # the whole workload against the HBM peak: algorithmic bytes of all
            # kernels of a step over the plain (untimed-kernel) step time
            "step_algorithmic_bytes": round(g["step_bytes"]),
            "step_algorithmic_GBps": round(g["step_bytes"] / (g["wall"] / args.steps) / 1e9, 1),
            "step_frac_of_hbm_peak": round(g["step_bytes"] / (g["wall"] / args.steps) / 1e9 / HBM_PEAK_GBS, 4),
            "hit_rate": round(g["h"], 4),
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
