"""A fresh checkout builds: the files git tracks (plus new, not ignored ones)
are copied to an empty directory, where ``__graft_entry__.build()`` and the
README's ``python -m hash_table_cache_amd.build`` must compile everything
from source and the package must then load its own freshly built library.
Cross-compilation only; no GPU involved."""

import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT


def checkout_files():
    try:
        out = subprocess.run(["git", "ls-files", "--cached", "--others", "--exclude-standard", "-z"], cwd=ROOT,
                             capture_output=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return None
    return [f for f in out.decode().split("\0") if f and os.path.isfile(os.path.join(ROOT, f))]


def test_fresh_checkout_builds_and_loads(tmp_path):
    files = checkout_files()
    if not files:
        pytest.skip("not a git work tree")
    for f in files:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy2(os.path.join(ROOT, f), dst)
    lib = tmp_path / "hash_table_cache_amd" / "_lib" / "libhkv.so"
    assert not lib.exists()
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    run = dict(cwd=tmp_path, env=env, capture_output=True, text=True, timeout=900)
    r = subprocess.run([sys.executable, "-m", "hash_table_cache_amd.build"], **run)
    assert r.returncode == 0, r.stderr[-3000:]
    assert lib.exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], **run)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-c",
                        "import hash_table_cache_amd as H; print(H._native.load()._name)"], **run)
    assert r.returncode == 0, r.stderr[-3000:]
    assert os.path.samefile(r.stdout.strip(), lib)
