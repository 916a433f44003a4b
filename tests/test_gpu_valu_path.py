"""GPU parity of the vector-ALU Q2_0 kernel where the matrix-core kernel would
normally run (K a multiple of 256 from 1024 up).

The kernel choice is read once per process from WQD_Q2_0_VALU, so the check
runs in a child process with that variable set.  The child compares against
the CPU oracle with the same acceptance rule and checks batched rows against
M=1 rows bit for bit.
"""
import os
import subprocess
import sys
import textwrap

import pytest

from parity import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import numpy as np
    import oracle
    from parity import check_parity, dev_u8, q2_0_gpu
    from weight_quantized_decode_block_amd import inputs as gen, wqd
    for (N, K, M) in [(5120, 5120, 8), (300, 2048, 3), (17, 1024, 9)]:
        A = gen.activations(21, K, M)
        codes, d = gen.q2_0_weights(21, N, K)
        Bd = dev_u8(wqd.q2_0_pack(codes, d))
        got = q2_0_gpu(A, Bd, N, K)
        check_parity(got, oracle.q2_0_gemv(A, codes, d), f"valu N={{N}} K={{K}} M={{M}}")
        for m in range(M):
            assert np.array_equal(got[m:m + 1], q2_0_gpu(A[m:m + 1], Bd, N, K, single=True)), m
        print("ok", N, K, M, flush=True)
""")


def test_forced_valu_kernel_parity():
    env = dict(os.environ, WQD_Q2_0_VALU="1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.count("ok") == 3
