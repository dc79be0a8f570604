"""GPU: the README's Python decode step runs as printed, and its output is finite."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    with open(os.path.join(ROOT, "README.md"), encoding="utf-8") as f:
        blocks = re.findall(r"```python\n(.*?)```", f.read(), re.S)
    assert blocks, "the README has no Python example"
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    out, lens = scope["out"], scope["lens"]
    assert out.shape == (3, 32, 128) and torch.isfinite(out.float()).all()
    assert lens.tolist() == [38, 501, 17]
