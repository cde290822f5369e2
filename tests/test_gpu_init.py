"""skinny_init from several host threads at once (include/skinny.h: call it
before any graph capture; idempotent; the compute calls read the device's
state without the init lock).  A fresh child process, so that the threads
race the first initialisation: every call returns SKINNY_OK and a GEMM
afterwards matches the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

_CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import moe_decode_skinny_amd as sk
import oracle, synthetic
from tests.helpers import assert_gemm_close, from_dev, to_dev
go = threading.Barrier(8)
status = []
def worker():
    go.wait()
    status.append(sk._lib.skinny_init(0))
ts = [threading.Thread(target=worker) for _ in range(8)]
for t in ts:
    t.start()
for t in ts:
    t.join(timeout=120)
assert status == [sk.SKINNY_OK] * 8, status
x, w = synthetic.gemm_inputs(N=1024, K=4096, seed=81)
y = torch.empty((8, 1024), dtype=torch.bfloat16, device="cuda")
sk.skinny_gemm_bf16(to_dev(x[:8]), to_dev(w), y, 0)
torch.cuda.synchronize()
assert_gemm_close(from_dev(y), oracle.gemm_bf16(x[:8], w, 8), "after concurrent init")
print("concurrent init ok", flush=True)
"""


def test_concurrent_first_init():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("child: 8 threads race skinny_init(0)", flush=True)
    res = subprocess.run([sys.executable, "-c", _CHILD, root], capture_output=True, text=True,
                         timeout=300, cwd=root)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    assert "concurrent init ok" in res.stdout
