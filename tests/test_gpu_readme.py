"""The usage example in README.md runs as written against the HIP library."""

import pathlib
import re

import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

README = pathlib.Path(__file__).resolve().parent.parent / "README.md"


def test_readme_usage_example_runs():
    text = README.read_text()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README has no python example"
    scope = {}
    exec(compile(blocks[0], "README.md example", "exec"), scope)
    found = scope["found"]
    assert bool(found.bool().all())  # every key inserted, then found (capacity far above the batch)
    assert int(scope["count"].item()) == 0  # re-inserting resident keys hands nothing back
    n = scope["keys"].numel()
    assert scope["outcomes"] == {"updated": 0, "inserted": n, "evicted": 0, "rejected": 0}
