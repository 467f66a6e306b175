"""CPU checks of bench.py's contract: the one-GPU exit, the algorithmic byte
counts behind its roofline figures, and the code hash that ties a committed
rocprofv3 summary to the kernel source it measured."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("dim,expected", [(64, 609.0), (32, 378.6)])
def test_find_bytes_match_the_derived_roofline(dim, expected):
    # one 128-byte digest line, 8-byte key in, half a false-positive key
    # compare, and for each hit (90 %) the 8-byte key plus the row read and
    # written: 141 + 8h + 8Dh bytes per key
    assert bench.find_bytes_per_key(dim, 0.9) == pytest.approx(expected)


def test_write_bytes_count_each_access_once():
    d = 64
    # resident key: key, line, false positives, candidate key, row in, score
    # in, row write, score write
    assert bench.probe_bytes_per_key(d, 1.0) == 8 + 128 + 4 + 8 + 4 * d + 8 + 4 * d + 8
    # missing key: key, line, false positives, chain link
    assert bench.probe_bytes_per_key(d, 0.0) == 8 + 128 + 4 + 8
    assert bench.assign_bytes_per_key(d) == 164 + 8 * d
    # owner kernel: the chain word of every key, nothing more without new keys
    assert bench.owner_bytes_per_key(d, 1.0, 1.0) == 4
    # an evicting new key adds the score column and one tied key
    assert (bench.owner_bytes_per_key(d, 0.0, 1.0) - bench.owner_bytes_per_key(d, 0.0, 0.0)) == 1024 + 8


def test_code_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SOURCE, encoding="utf-8").read()
    h0 = bench.kernel_code_sha256()
    commented = tmp_path / "k.hip"
    commented.write_text("// a comment\n/* block\n comment */\n" + src.replace(";", ";  ") + "\n\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(commented))
    assert bench.kernel_code_sha256() == h0
    changed = tmp_path / "k2.hip"
    changed.write_text(src.replace("kBlock = 256", "kBlock = 512", 1))
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(changed))
    assert bench.kernel_code_sha256() != h0


def test_cold_runs_report_medians_of_fresh_processes(monkeypatch, capsys):
    """--cold-runs starts one child process per run (this process never
    touches the GPU) and reports the median of each per-lambda rate."""
    finds = [[10.0, 9.0], [12.0, 8.0], [11.0, 10.0]]
    calls = []

    class Done:
        returncode = 0
        stderr = ""

        def __init__(self, k):
            per = {"0.5": {"find_bkvs": finds[k][0], "upsert_bkvs": 5.0 + k},
                   "1.0": {"find_bkvs": finds[k][1], "upsert_bkvs": 4.0}}
            self.stdout = "log line\n" + json.dumps({"value": 6.0 + k, "detail": {"per_lambda": per}})

    def fake_run(cmd, **kw):
        calls.append(cmd)
        return Done(len(calls) - 1)

    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--cold-runs", "3", "--dim", "32"])
    bench.main()
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert len(calls) == 3 and all("--dim" in c and c[c.index("--dim") + 1] == "32" for c in calls)
    assert all("--cold-runs" not in c for c in calls)
    assert out["per_lambda_median"]["0.5"]["find_bkvs"] == 11.0
    assert out["per_lambda_median"]["1.0"]["find_bkvs"] == 9.0
    assert out["per_lambda_median"]["0.5"]["upsert_bkvs"] == 6.0
    assert out["combined_bkvs_median"] == 7.0
    assert out["find_lambda_variation"] == pytest.approx(round((11.0 - 9.0) / 11.0, 4))


def test_json_line_carries_the_contract_fields(monkeypatch, capsys):
    """With the GPU work replaced by canned results, main() prints one JSON
    line with every field the benchmark contract requires: value as keys over
    wall time, the roofline object of the dominant kernel (its traffic from
    the committed rocprofv3 summary of the same kernel code and workload) and
    the CPU oracle baseline."""
    kern = {"find": dict(avg_ms=0.117, achieved_GBps=5400.0, frac=0.675, bytes_per_launch=638_000_000),
            "upsert_probe": dict(avg_ms=0.14, achieved_GBps=4660.0, frac=0.5825, bytes_per_launch=653_000_000)}
    g = dict(total_keys=8 * (1 << 20) * 20, wall=20 * 1.2e-3, dominant="upsert_probe", kernels=kern,
             wall_timed_kernels=20 * 1.25e-3, gpu_busy_frac=0.95, detail={}, find_var=0.02, insert_new=None,
             extra_ops={}, step_bytes=5.6e9, h=0.9)
    monkeypatch.setattr(bench, "run_gpu", lambda args: dict(g))
    monkeypatch.setattr(bench, "copy_bandwidth", lambda: 5000.0)
    monkeypatch.setattr(bench, "pattern_ceiling", lambda dim: None)
    g["cpu_sample"] = dict(lam=0.5, li=0, warmup=3, batches=[])
    monkeypatch.setattr(bench, "run_cpu_baseline",
                        lambda args, sample: dict(value=0.004, secs=8.0, total=14.0, fill_s=20.0, steps=6, lam=0.5,
                                                  cap=1 << 26, batch=1 << 20, core=7, find_bkvs=0.005,
                                                  upsert_bkvs=0.0015, cpu_model="x", nproc=8, allowed=8))
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 3 and d["higher_is_better"] is True
    assert d["value"] == pytest.approx(8 * (1 << 20) / 1.2e-3 / 1e9, rel=1e-3)
    assert d["ms_per_step"] == pytest.approx(1.2)
    assert "workload" in d["config"] and "model" not in d["config"]
    r = d["roofline"]
    assert r["kernel"] == "upsert_probe" and r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["traffic"] == bench.profiled_traffic("upsert_probe", 64, 26)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["unit"] == d["unit"] and c["sample"]


def test_launch_cv_reads_the_library_record():
    """The library's per-kernel record is (launches, total_ms, max_ms, min_ms,
    sum of squares, median_ms); three launches of 1, 2 and 3 ms."""
    rec = (3, 6.0, 3.0, 1.0, 14.0, 2.0)
    assert bench.launch_cv(rec) == round((14.0 / 3 - 4.0) ** 0.5 / 2.0, 4)
