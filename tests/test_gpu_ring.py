"""GPU parity of the layer ring (skinny_gemm_bf16_ring) through the C ABI.

The ring runs `count` independent GEMMs of one shape in one persistent
launch, streaming the next item's weights while it finishes the current one
(unpooler page, module description: weights before the dependency wait,
activations after).  Each item must
  - match the oracle within |err| <= 2^-7 |ref| + 2^-10 rms(ref),
  - be bitwise identical to the single-call GEMM at the ring's launch shape
    (the per-tile arithmetic and summation order are the same),
  - be reproducible bit for bit, and bit-exact on integer inputs,
and nothing outside the y buffers may be written.
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
POISON = -12345.0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _items(count, N, K, seed, integer=False, M=16):
    xs, ws = [], []
    for i in range(count):
        if integer:
            x, w = synthetic.exact_integer_inputs(M=M, N=N, K=K, seed=seed + i)
        else:
            x, w = synthetic.gemm_inputs(N=N, K=K, seed=seed + i)
        xs.append(x)
        ws.append(w)
    return xs, ws


def _ring(sk, xs_bits, ws_bits, M, launch=None, reps=1):
    """Run the ring; returns the list of y bit arrays (of the last rep) and
    checks the guard regions around every y."""
    import torch

    count = len(ws_bits)
    N, K = ws_bits[0].shape
    xs = [to_dev(x[:M]) for x in xs_bits]
    ws = [to_dev(w) for w in ws_bits]
    guard = 64
    stride = M * N + 2 * guard
    buf = torch.full((count * stride,), POISON, dtype=torch.bfloat16, device="cuda")
    ys = [buf[i * stride + guard:i * stride + guard + M * N].view(M, N) for i in range(count)]
    outs = []
    for _ in range(reps):
        if launch is None:
            sk.skinny_gemm_bf16_ring(xs, ws, ys)
        else:
            sk.skinny_gemm_bf16_ring_launch(xs, ws, ys, launch)
        torch.cuda.synchronize()
        outs.append([from_dev(y).copy() for y in ys])
    b = from_dev(buf).reshape(count, stride)
    pb = from_dev(torch.tensor([POISON], dtype=torch.bfloat16))[0]
    assert np.all(b[:, :guard] == pb) and np.all(b[:, guard + M * N:] == pb), "write outside y"
    for o in outs[1:]:
        for i in range(count):
            assert np.array_equal(o[i], outs[0][i]), f"item {i} not reproducible"
    return outs[-1]


def _single(sk, x_bits, w_bits, M, launch):
    import torch

    N = w_bits.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sk.skinny_gemm_bf16_launch(to_dev(x_bits[:M]), to_dev(w_bits), y, _as_single(sk, launch))
    torch.cuda.synchronize()
    return from_dev(y)


def _ring_launches(sk, M, N, K):
    """Ring launch candidates of every family with splits = 1: DOT2 rows
    2..16 x chunks 1, 2, 4, MFMA 4x4 rows 4, 8 x chunks 4, 8 and MFMA 1, 2, 4
    tiles x chunks 1..16 x accs 1, 2 (the ring validator decides which it has
    kernels for)."""
    out = []
    for rows in (2, 4, 8, 16):
        for chunks in (1, 2, 4):
            out.append(sk.Launch(0, 1, -(-K // (512 * chunks)), chunks, 1, rows))
    for rows in (4, 8):
        for chunks in (4, 8):
            out.append(sk.Launch(sk.SKINNY_PATH_MFMA_4X4, 1, -(-K // (128 * chunks)), chunks, 1,
                                 rows))
    for path in (sk.SKINNY_PATH_MFMA, sk.SKINNY_PATH_MFMA_LDS):
        for rows in (16, 32, 64):
            for chunks in (1, 2, 4, 8, 16):
                for accs in (1, 2):
                    out.append(sk.Launch(path, 1, rows // 16 * -(-K // (32 * chunks)), chunks,
                                         accs, rows))
    return [l for l in out if N % l.rows == 0]


def _as_single(sk, launch):
    """The single-call launch with the ring launch's arithmetic (the staged
    MFMA ring computes what the plain MFMA kernel does)."""
    if launch.path == sk.SKINNY_PATH_MFMA_LDS:
        return launch._replace(path=sk.SKINNY_PATH_MFMA)
    return launch


def _single_ok(sk, M, N, K, launch):
    return sk.skinny_launch_unsupported(M, N, K, _as_single(sk, launch)) is None


@pytest.mark.parametrize("M", [1, 2, 3, 8, 9, 16])
def test_ring_unpooler_parity(gpu_lib, M):
    """Six unpooler-shard items (N=1024, K=4096), each with its own x and W."""
    N, K = 1024, 4096
    xs, ws = _items(6, N, K, seed=100)
    launch = gpu_lib.skinny_ring_choose(M, N, K, len(ws))
    _say(f"ring unpooler M={M} {launch}")
    ys = _ring(gpu_lib, xs, ws, M, reps=3)
    for i, (x, w, y) in enumerate(zip(xs, ws, ys)):
        assert_gemm_close(y, oracle.gemm_bf16(x[:M], w, THREADS), f"item {i}")
        if _single_ok(gpu_lib, M, N, K, launch.gemm):
            assert np.array_equal(y, _single(gpu_lib, x, w, M, launch.gemm)), \
                f"item {i} != single call"


def _walks(groups, count):
    """(segment, workgroups) pairs: one block per visit and whole items per
    visit, with one workgroup, three (items interleave across workgroups)
    and one per segment."""
    out = []
    for seg in sorted({1, 2, groups}):
        if groups % seg:
            continue
        segs = count * groups // seg
        for wg in sorted({1, 3, groups // seg, segs}):
            if 1 <= wg <= segs:
                out.append((seg, wg))
    return out


@pytest.mark.parametrize("M,N,K", [(1, 64, 1024), (3, 48, 1000), (7, 128, 2056), (16, 32, 520),
                                   (4, 16, 8), (12, 64, 1000), (16, 32, 8000), (5, 64, 6000)])
def test_ring_every_launch_and_walk(gpu_lib, M, N, K):
    """Every compiled ring variant the validator accepts on small ragged
    shapes, under several tile walks (segment length and workgroup count)."""
    count = 5
    xs, ws = _items(count, N, K, seed=200)
    refs = [oracle.gemm_bf16(x[:M], w, THREADS) for x, w in zip(xs, ws)]
    tried = 0
    for g in _ring_launches(gpu_lib, M, N, K):
        groups = N // g.rows
        single = _single_ok(gpu_lib, M, N, K, g)
        singles = [_single(gpu_lib, xs[i], ws[i], M, g) for i in range(count)] if single else None
        for seg, wg in _walks(groups, count):
            launch = gpu_lib.RingLaunch(g, seg, wg)
            reason = gpu_lib.skinny_ring_launch_unsupported(M, N, K, count, launch)
            if reason is not None:
                assert "kernel" in reason or "waves" in reason, reason
                break
            tried += 1
            _say(f"ring M={M} N={N} K={K} {launch}")
            ys = _ring(gpu_lib, xs, ws, M, launch=launch)
            for i in range(count):
                assert_gemm_close(ys[i], refs[i], f"{launch} item {i}")
                if single:
                    assert np.array_equal(ys[i], singles[i]), f"{launch} item {i} != single call"
    assert tried


@pytest.mark.parametrize("path", ["dot2", "mfma_4x4", "mfma_lds"])
def test_ring_xcd_local_walk(gpu_lib, path):
    """19 items: in the XCD-local order with a workgroup count divisible by 8
    the first 16 items' segments are dealt XCD by XCD and the last 3 follow
    item-major; with other counts, and in the item-major order, all slots are
    item-major.  Every item must be bitwise the single call at the same
    launch under every walk and order."""
    M, N, K, count = 12, 128, 1032, 19
    g = {"dot2": gpu_lib.Launch(0, 1, 3, 1, 1, 4),
         "mfma_4x4": gpu_lib.Launch(3, 1, 3, 4, 1, 8),
         "mfma_lds": gpu_lib.Launch(2, 1, 9, 4, 1, 16)}[path]
    xs, ws = _items(count, N, K, seed=250)
    singles = [_single(gpu_lib, xs[i], ws[i], M, g) for i in range(count)]
    for i in (0, count - 1):
        assert_gemm_close(singles[i], oracle.gemm_bf16(xs[i][:M], ws[i], THREADS), f"item {i}")
    groups = N // g.rows
    for seg in (1, 2, groups):
        for wg in (8, 16, 24, 12, 7):
            for order in (gpu_lib.SKINNY_RING_XCD_LOCAL, gpu_lib.SKINNY_RING_ITEM_MAJOR):
                launch = gpu_lib.RingLaunch(g, seg, min(wg, count * groups // seg), order)
                assert gpu_lib.skinny_ring_launch_unsupported(M, N, K, count, launch) is None
                _say(f"xcd walk {path} {launch}")
                ys = _ring(gpu_lib, xs, ws, M, launch=launch)
                for i in range(count):
                    assert np.array_equal(ys[i], singles[i]), f"{launch} item {i}"


def test_ring_max_count(gpu_lib):
    """64 items (the most one call takes) on a small ragged shape."""
    M, N, K = 4, 64, 1032
    xs, ws = _items(64, N, K, seed=300)
    _say("ring count=64")
    ys = _ring(gpu_lib, xs, ws, M)
    for i in range(64):
        assert_gemm_close(ys[i], oracle.gemm_bf16(xs[i][:M], ws[i], THREADS), f"item {i}")


@pytest.mark.parametrize("M,N,K,count", [(4, 65536, 64, 3), (16, 49152, 520, 2),
                                         (1, 8192, 1024, 4), (8, 8192, 1024, 3),
                                         (16, 8192, 1024, 2), (1, 512, 8192, 4),
                                         (8, 512, 8192, 4), (16, 512, 8192, 3),
                                         (1, 4096, 8192, 2), (8, 4096, 8192, 2),
                                         (16, 4096, 8192, 2)])
def test_ring_shard_shapes(gpu_lib, M, N, K, count):
    """The o_proj and pooler shard shapes."""
    xs, ws = _items(count, N, K, seed=400)
    launch = gpu_lib.skinny_ring_choose(M, N, K, count)
    _say(f"ring M={M} N={N} K={K} {launch}")
    ys = _ring(gpu_lib, xs, ws, M)
    for i in range(count):
        assert_gemm_close(ys[i], oracle.gemm_bf16(xs[i][:M], ws[i], THREADS), f"item {i}")


@pytest.mark.parametrize("M", [1, 2, 5, 8, 16])
def test_ring_exact_integer_inputs_bit_exact(gpu_lib, M):
    N, K = 256, 2048
    xs, ws = _items(4, N, K, seed=500 + M, integer=True)
    _say(f"ring integer M={M}")
    ys = _ring(gpu_lib, xs, ws, M)
    for i in range(4):
        assert np.array_equal(ys[i], oracle.gemm_bf16(xs[i][:M], ws[i], THREADS)), f"item {i}"


@pytest.mark.parametrize("M,N,K", [(8, 1024, 4096), (16, 1024, 4096), (16, 8192, 1024),
                                   (16, 512, 8192), (8, 4096, 8192), (16, 4096, 8192)])
def test_ring_sixty_layer_weight_ring(gpu_lib, M, N, K):
    """A 60-layer weight ring of shard weights (more than the caches hold) as
    one 60-item call at the ring chooser's launch (the bench's launches:
    XCD-local slots), each item with its own x; sampled oracle positions on
    every layer, full check on two."""
    import torch

    ring = synthetic.device_weight_ring(60, N, K, "cuda")
    _say(f"ring over 60 device layers M={M} N={N} K={K} {gpu_lib.skinny_ring_choose(M, N, K, 60)}")
    xs_bits = [synthetic.gemm_inputs(N=16, K=K, seed=600 + i)[0][:M] for i in range(60)]
    xs = [to_dev(x) for x in xs_bits]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in ring]
    gpu_lib.skinny_gemm_bf16_ring(xs, ring, ys)
    torch.cuda.synchronize()
    rng = np.random.default_rng(601)
    rows = rng.integers(0, M, 64)
    cols = rng.integers(0, N, 64)
    tile = gpu_lib.skinny_ring_choose(M, N, K, 60).gemm
    for layer in range(60):
        x_bits = xs_bits[layer]
        w_bits = from_dev(ring[layer])
        y = from_dev(ys[layer])
        if layer in (0, 59):
            assert_gemm_close(y, oracle.gemm_bf16(x_bits, w_bits, THREADS), f"layer {layer}")
        if layer in (0, 31, 59) and _single_ok(gpu_lib, M, N, K, tile):
            assert np.array_equal(y, _single(gpu_lib, x_bits, w_bits, M, tile)), f"layer {layer}"
        ref, exact = oracle.gemm_bf16_sampled(x_bits, w_bits, rows, cols)
        r = oracle.bf16_value(ref)
        g = oracle.bf16_value(y[rows, cols])
        scale = np.sqrt(np.mean(exact ** 2))  # rms of y estimated from the samples
        assert np.all(np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 2.0 ** -10 * scale), f"layer {layer}"
    # the same launch again: every item bitwise as before
    first = [from_dev(y) for y in ys]
    for y in ys:
        y.fill_(0)
    gpu_lib.skinny_gemm_bf16_ring(xs, ring, ys)
    torch.cuda.synchronize()
    for layer in range(60):
        assert np.array_equal(from_dev(ys[layer]), first[layer]), f"layer {layer} not reproducible"


def test_ring_graph_capture_replay(gpu_lib):
    """The ring recorded in a HIP graph and replayed with new activations and
    eager work between replays."""
    import torch

    M, N, K, count = 4, 1024, 4096, 3
    xs_bits, ws_bits = _items(count, N, K, seed=700)
    alt, _ = _items(count, 16, K, seed=710)
    xs = [to_dev(x[:M]) for x in xs_bits]
    ws = [to_dev(w) for w in ws_bits]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(count)]
    gpu_lib.skinny_gemm_bf16_ring(xs, ws, ys)
    torch.cuda.synchronize()
    eager = [from_dev(y).copy() for y in ys]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gpu_lib.skinny_gemm_bf16_ring(xs, ws, ys)
    torch.cuda.synchronize()
    for rep in range(4):
        _say(f"ring graph replay {rep}")
        for y in ys:
            y.fill_(7.0)
        src = xs_bits if rep % 2 == 0 else alt
        for x, b in zip(xs, src):
            x.copy_(to_dev(b[:M]))
        g.replay()
        torch.cuda.synchronize()
        for i in range(count):
            if rep % 2 == 0:
                assert np.array_equal(from_dev(ys[i]), eager[i])
            else:
                assert_gemm_close(from_dev(ys[i]),
                                  oracle.gemm_bf16(alt[i][:M], ws_bits[i], THREADS), "replay")
