"""The usage example of the repository's README runs as written (on the MI355X): the code block
under its "Using it" heading is executed, and every output it produces must be finite."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_example_runs():
    text = open(README).read()
    section = text.split("## Using it", 1)[1]
    code = re.search(r"```python\n(.*?)```", section, re.S).group(1)
    env = {}
    exec(compile(code, "README example", "exec"), env)
    torch.cuda.synchronize()
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        for t in env[name].values():
            assert torch.isfinite(t).all(), name
    assert len(env["tiles"]) == 64
