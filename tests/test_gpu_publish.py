"""GPU parity of the zero-copy publish (skinny_gemm_bf16_publish) through the
C ABI, on one GPU.

In the unpooler page's zero-copy epilogue, the kernel that stores y also
copies it into the calling rank's slot of the mailbox read at the following
boundary ([3 stages][tp][capacity][width] BF16), writing -0.0 as +0.0 (the pooler_gather page: -0.0 is the mailbox's sentinel) and
sets the active-stage word, or takes the stage from a ticket's upper half and
stores no word.  Here y must match the oracle GEMM within the GEMM tolerance
and be bitwise equal to the plain call at the same launch; the mailbox and
the stage state must equal the oracle's publish of the GPU's y, bit for bit,
with every byte outside the slot untouched.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests.helpers import assert_gemm_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)
POISON_BITS = 0x1234  # a bf16 pattern no publish writes here


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _i32(vals):
    import torch

    return torch.tensor(vals, dtype=torch.int32, device="cuda")


def _mailbox(tp, capacity, width):
    import torch

    host = np.full((3, tp, capacity, width), POISON_BITS, dtype=np.uint16)
    return host, torch.from_numpy(host.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _publish(sk, x_bits, w_bits, M, launch=None, tp=4, rank=2, capacity=16, stage=None,
             ticket=None):
    import torch

    N, K = w_bits.shape
    host_mb, mb = _mailbox(tp, capacity, N)
    st = None if stage is None else _i32(stage)
    tk = None if ticket is None else _i32(ticket)
    x = to_dev(x_bits[:M])
    w = to_dev(w_bits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sk.skinny_gemm_bf16_publish(x, w, y, mb, rank, stage_state=st, ticket=tk, launch=launch)
    torch.cuda.synchronize()
    y_bits = from_dev(y)
    # the oracle's publish of the GPU's y into a host copy of the mailbox
    want_st = None if stage is None else np.array(stage, dtype=np.int32)
    want_tk = None if ticket is None else np.array(ticket, dtype=np.int32)
    used = oracle.mailbox_publish(y_bits, host_mb, rank, stage_state=want_st, ticket=want_tk)
    assert np.array_equal(from_dev(mb).reshape(host_mb.shape), host_mb), "mailbox differs"
    if st is not None:
        assert st.cpu().numpy().tolist() == want_st.tolist(), "stage state differs"
    if tk is not None:
        assert tk.cpu().numpy().tolist() == list(ticket), "ticket written"
    return y_bits, used


def _plain(sk, x_bits, w_bits, M, launch):
    import torch

    N = w_bits.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    if launch is None:
        sk.skinny_gemm_bf16(x, w, y, 0)
    else:
        sk.skinny_gemm_bf16_launch(x, w, y, launch)
    torch.cuda.synchronize()
    return from_dev(y)


def _launches(sk, M, N, K):
    """The chooser's launch and one launch per store site: DOT2, MFMA and
    MFMA 4x4 with one split (the GEMM kernel stores y), DOT2 and MFMA with
    splits (the split-reduce kernel does), and MFMA 4x4 with 2 and 4 splits
    (the last workgroup of each output group to finish does), and MFMA 4x4
    with two token groups, without and with splits (from M = 5)."""
    out = [None,
           sk.Launch(0, 1, -(-K // 1024), 2, 1, 4),
           sk.Launch(1, 1, -(-K // 256), 8, 1, 16),
           sk.Launch(3, 1, -(-K // 512), 4, 1, 4),
           sk.Launch(0, 4, -(-K // (4 * 512)), 1, 1, 4),
           sk.Launch(1, 2, 2 * -(-K // (2 * 32 * 8)), 8, 2, 32),
           sk.Launch(3, 2, -(-K // (2 * 512)), 4, 1, 4),
           sk.Launch(3, 4, -(-K // (4 * 512)), 4, 1, 8),
           sk.Launch(3, 1, -(-K // 512), 4, 2, 4),
           sk.Launch(3, 2, -(-K // (2 * 512)), 4, 2, 4)]
    return [l for l in out if l is None or sk.skinny_launch_unsupported(M, N, K, l) is None]


@pytest.mark.parametrize("M", [1, 5, 16])
def test_publish_every_store_site(gpu_lib, M):
    N, K = 1024, 4096
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=40)
    ref = oracle.gemm_bf16(x[:M], w, THREADS)
    launches = _launches(gpu_lib, M, N, K)
    assert len(launches) >= 7
    for l in launches:
        _say(f"publish M={M} {l}")
        y, used = _publish(gpu_lib, x, w, M, launch=l, stage=[1, 7])
        assert used == 1
        assert_gemm_close(y, ref, f"publish {l}")
        assert np.array_equal(y, _plain(gpu_lib, x, w, M, l)), f"{l}: y differs from the plain call"


@pytest.mark.parametrize("stage", [0, 2])
def test_publish_stage_state_shapes(gpu_lib, stage):
    """Other mailbox geometries: one rank, the last rank, M == capacity."""
    N, K, M = 512, 1000, 3
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=41)
    for tp, rank, cap in ((1, 0, 3), (8, 7, 5), (3, 1, 16)):
        _say(f"publish stage={stage} tp={tp} rank={rank} capacity={cap}")
        y, used = _publish(gpu_lib, x, w, M, tp=tp, rank=rank, capacity=cap, stage=[stage, -1])
        assert used == stage
        assert_gemm_close(y, oracle.gemm_bf16(x[:M], w, THREADS), "publish shapes")


def test_publish_ticket(gpu_lib):
    """With a ticket the stage is its upper half; no stage word is written and
    a stage state given beside it is not touched."""
    N, K, M = 1024, 4096, 8
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=42)
    for l in _launches(gpu_lib, M, N, K):
        _say(f"publish ticket {l}")
        y, used = _publish(gpu_lib, x, w, M, launch=l, stage=[0, 9], ticket=[(2 << 16) | 3])
        assert used == 2


@pytest.mark.parametrize("stage,ticket", [([3, 9], None), ([-1, 9], None), (None, [3 << 16])])
def test_publish_stage_outside_range_writes_nothing(gpu_lib, stage, ticket):
    N, K, M = 1024, 4096, 4
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=43)
    for l in _launches(gpu_lib, M, N, K):
        _say(f"publish out of range {stage} {ticket} {l}")
        y, used = _publish(gpu_lib, x, w, M, launch=l, stage=stage, ticket=ticket)
        assert used == -1
        assert_gemm_close(y, oracle.gemm_bf16(x[:M], w, THREADS), "y still stored")


def test_publish_negative_zero_stored_as_positive_zero(gpu_lib):
    """y entries that round to -0.0: a product -2^-70 * 2^-70 = -2^-140 per
    output (FP32 subnormal, kept by the kernels), below half the smallest
    bf16 subnormal.  y must be the oracle's -0.0 bit for bit and the mailbox
    must hold +0.0 there (the oracle publish of the GPU's y, bit for bit)."""
    N, K, M = 256, 512, 4
    x = np.zeros((16, K), dtype=np.uint16)
    w = np.zeros((N, K), dtype=np.uint16)
    x[:, 0] = oracle.bf16_round(-(2.0 ** -70))
    w[:, 0] = oracle.bf16_round(2.0 ** -70)
    w[::2, 1] = oracle.bf16_round(1.0)        # even features add a -0.0 * 1.0 term
    x[:, 1] = 0x8000                          # -0.0 times 1.0 = -0.0
    ref = oracle.gemm_bf16(x[:M], w, THREADS)
    assert np.all(ref == 0x8000)              # the exact sums round to -0.0
    for l in _launches(gpu_lib, M, N, K):
        _say(f"publish -0.0 {l}")
        y, _ = _publish(gpu_lib, x, w, M, launch=l, stage=[0, 5])
        assert np.array_equal(y, ref), f"{l}: y is not -0.0 everywhere"
        assert np.array_equal(_plain(gpu_lib, x, w, M, l), ref)


def test_publish_stage_read_when_the_graph_replays(gpu_lib):
    """The stage is read on the device: a captured publish replayed after the
    stage state changes writes the slot of the new stage."""
    import torch

    N, K, M = 1024, 4096, 8
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=44)
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    host_mb, mb = _mailbox(2, 8, N)
    st = _i32([0, 0])
    gpu_lib.skinny_gemm_bf16_publish(x, w, y, mb, 1, stage_state=st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gpu_lib.skinny_gemm_bf16_publish(x, w, y, mb, 1, stage_state=st)
    torch.cuda.synchronize()
    want_st = np.array([0, 0], dtype=np.int32)
    y_bits = from_dev(y)
    oracle.mailbox_publish(y_bits, host_mb, 1, stage_state=want_st)
    for stage in (1, 2, 0, 2):
        _say(f"graph replay, stage {stage}")
        st.copy_(_i32([stage, 9]))
        want_st[:] = [stage, 9]
        g.replay()
        torch.cuda.synchronize()
        oracle.mailbox_publish(y_bits, host_mb, 1, stage_state=want_st)
        assert np.array_equal(from_dev(y), y_bits)
        assert np.array_equal(from_dev(mb).reshape(host_mb.shape), host_mb)
        assert st.cpu().numpy().tolist() == [stage, stage]
