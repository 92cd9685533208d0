"""The C ABI driven from plain C (tests/c/z1_c_abi_test.c, built by
__graft_entry__.build()): four steps -- an accumulation call per
micro-batch, all slots in one z1_accum_grads_range call, a packed-layout
plan, and AdamW through a one-row schedule -- each bit-exact against the
oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "z1_c_abi_test")


def test_c_program_step_bitexact():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "build the C test first: python __graft_entry__.py build"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "bit-exact" in r.stdout, (r.returncode, r.stdout, r.stderr)
