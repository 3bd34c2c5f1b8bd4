"""The Python usage example in README.md runs as written."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README has no python example"
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    import torch
    torch.cuda.synchronize()
    for name in ("o", "o_w", "dq", "dk", "dv", "o_dec", "o8"):
        assert torch.isfinite(env[name].float()).all(), name
    assert env["o_dec"].shape == (4, 1, 32, 128)
