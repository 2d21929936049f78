"""The Python example of README.md runs as written (on the GPU), so the
documentation cannot drift from the binding."""

import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_example_runs(gpu):
    text = open(README).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1, "README holds one Python example"
    print("[readme] running the README example", flush=True)
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    for name in ("out", "dq", "dk", "dv"):
        t = scope[name]
        assert torch.isfinite(t.float()).all(), name
    assert not torch.isnan(scope["lse"]).any()   # -inf marks a row with no live tile
    assert scope["out"].shape == scope["q"].shape
