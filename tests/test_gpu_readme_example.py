"""The usage example of README.md, run as written (its first python block)."""
import os
import re

import pytest

from tests.parity import say

pytestmark = pytest.mark.gpu


def test_readme_usage_example_runs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")
    with open(path) as f:
        text = f.read()
    m = re.search(r"```python\n(.*?)```", text, re.S)
    assert m, "README.md has no python block"
    say("README usage example")
    scope = {}
    exec(compile(m.group(1), "README.md", "exec"), scope)
    torch.cuda.synchronize()
    T, H, d = scope["T"], scope["H"], scope["d"]
    assert scope["o"].shape == (T, H, d) and scope["dq"].shape == (T, H, d)
    assert scope["og"].shape == (T, H, d) and scope["dh0"].shape == (scope["B"], H, d, d)
    for name in ("o", "dq", "dk", "dv", "og", "dqn", "dkn", "dvg", "dg", "dbeta"):
        assert bool(torch.isfinite(scope[name].float()).all()), name
