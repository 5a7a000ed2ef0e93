"""A process's first few-row and tiled MLP calls captured into HIP graphs.

The library allocates nothing: split-K partials live in the caller's
workspace, so even the first call of a process (no warm-up) can be captured,
and every replay equals the eager result bit for bit.  The capture must be
the process's first use of the library, so the cases run in a child process
(tests/graph_first_call.py) with its own time limit."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_first_calls_captured_in_graphs():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU")
    p = subprocess.run([sys.executable, os.path.join(HERE, "graph_first_call.py")], capture_output=True, text=True,
                       timeout=300)
    print(p.stdout, p.stderr[-4000:], flush=True)
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert p.stdout.count(": ok") == 4
