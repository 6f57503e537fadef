"""The library from a plain C program: tests/native/allreduce_worked_example.c
(built by build() with gcc against include/vrcomm.h) runs the Symmetric page's
AllReduce example, 4 ranks x 1 Mi fp32 filled with the rank value, and checks
every element (6.0) and every completion signal itself."""
import os
import subprocess

import pytest

from conftest import ROOT
from gpu_util import say

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(ROOT, "tests", "native", "allreduce_worked_example")


def test_c_client_runs_the_worked_example():
    assert os.path.exists(CLIENT), "build() compiles the C client"
    say("C client: 4 ranks x 1 Mi fp32 AllReduce, every element 6.0")
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok: 4 ranks"), r.stdout
