"""The plain C client of the C ABI (tests/c_client.c, built by
__graft_entry__.build()) on the GPU: include/gq.h used from C11 with the HIP
runtime's C interface, exact closed-form results for gq_matvec, gq_matmul
and gq_dequant, and host-side rejections."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gq_c_client")


def test_c_client():
    assert os.path.exists(CLIENT), "tests/gq_c_client is built by __graft_entry__.build()"
    print("[c client] running tests/gq_c_client", flush=True)
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client ok" in r.stdout
