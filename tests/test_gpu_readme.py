"""The Python example in README.md runs as written and produces finite
outputs on every written row (the documentation stays in step with the
binding)."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_example_runs():
    text = open(README, encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    o, lse = env["o"], env["lse"]
    assert env["nnz"] > 0
    assert not torch.isnan(o.float()).any()
    assert not torch.isnan(lse).any()
