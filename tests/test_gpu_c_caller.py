"""A plain C99 caller of libpagedattn on the GPU.

tests/c/abi_check.c uses nothing but include/pagedattn.h and the HIP
runtime's C API: it fills float32 pools, appends one token per sequence with
pa_kv_append and decodes with pa_decode (with a workspace, then without), and
checks results with closed forms - a one-token context returns its V row
exactly, a zero query returns the mean of the visible V rows, the appended
rows land at their slots bit for bit.  __graft_entry__.build() links it.
"""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")


def test_c_caller_decodes_a_step():
    if not os.path.exists(EXE):
        pytest.fail("tests/c/abi_check is not built: run __graft_entry__.build()")
    proc = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                          timeout=90)
    assert proc.returncode == 0, proc.stdout
    assert "abi_check ok" in proc.stdout
