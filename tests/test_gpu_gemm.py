"""GPU parity of skinny_gemm_bf16 against the oracle, through the C ABI.

Workloads (synthetic, seeded; the shard shapes of the three API pages):
  unpooler shard  N=1024, K=4096 (unpooler page, module description)
  o_proj shard    N=8192, K=1024 (oproj.batt page, OProjection)
  pooler shard    N=512,  K=8192 and the full pooler N=4096, K=8192
                  (pooler_gather page, module description)
x ~ N(0, 1), W ~ N(0, 1/K).  Acceptance: |err| <= 2^-7 |ref| + 2^-10 rms(ref)
per element (tests/helpers.py), bitwise determinism per launch shape
(unpooler page, module description: the order of the partial sums is a
function of the launch shape alone), and
bit-exactness on integer inputs whose sums are exact in any order.
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


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(sk, x_bits, w_bits, M, splits=0, launch=None, poison=True):
    import torch

    N, K = w_bits.shape
    x = to_dev(x_bits[:M])
    w = to_dev(w_bits)
    # y sits inside a larger buffer whose other bytes are poisoned; rows >= M
    # and the guard regions must come back untouched.
    guard = 64
    buf = torch.full((2 * guard + 16 * N,), -12345.0, dtype=torch.bfloat16, device="cuda")
    y = buf[guard:guard + M * N].view(M, N)
    if launch is None:
        sk.skinny_gemm_bf16(x, w, y, splits)
    else:
        sk.skinny_gemm_bf16_launch(x, w, y, launch)
    torch.cuda.synchronize()
    b = from_dev(buf)
    poison_bits = from_dev(torch.tensor([-12345.0], dtype=torch.bfloat16))[0]
    if poison:
        assert np.all(b[:guard] == poison_bits) and np.all(b[guard + M * N:] == poison_bits), \
            "write outside y"
    return from_dev(y)


@pytest.fixture(scope="module")
def unpooler_inputs():
    return synthetic.gemm_inputs(N=1024, K=4096, seed=0)


def test_unpooler_m1_s1(gpu_lib, unpooler_inputs):
    x, w = unpooler_inputs
    _say("unpooler M=1 N=1024 K=4096 S=1")
    y = _run(gpu_lib, x, w, 1, splits=1)
    assert_gemm_close(y, oracle.gemm_bf16(x[:1], w, THREADS), "unpooler M=1 S=1")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("splits", [0, 1, 2, 4])
def test_unpooler_sweep_parity_and_determinism(gpu_lib, unpooler_inputs, M, splits):
    """splits=0 is the chooser's launch, the one bench.py times."""
    x, w = unpooler_inputs
    _say(f"unpooler M={M} S={splits}")
    ref = oracle.gemm_bf16(x[:M], w, THREADS)
    first = _run(gpu_lib, x, w, M, splits=splits)
    assert_gemm_close(first, ref, f"unpooler M={M} S={splits}")
    for _ in range(9):
        again = _run(gpu_lib, x, w, M, splits=splits, poison=False)
        assert np.array_equal(again, first), "not bitwise reproducible"


def _parity_and_repeats(sk, x, w, M, what, repeats=10):
    """The chooser's launch (the one bench.py times) against the oracle, then
    bitwise equal over `repeats` runs in all."""
    first = _run(sk, x, w, M)
    assert_gemm_close(first, oracle.gemm_bf16(x[:M], w, THREADS), what)
    for _ in range(repeats - 1):
        assert np.array_equal(_run(sk, x, w, M, poison=False), first), \
            f"{what}: not bitwise reproducible"


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_oproj_shard(gpu_lib, M):
    x, w = synthetic.gemm_inputs(N=8192, K=1024, seed=3)
    _say(f"o_proj M={M}")
    _parity_and_repeats(gpu_lib, x, w, M, f"o_proj M={M}")


@pytest.mark.parametrize("N", [512, 4096])
@pytest.mark.parametrize("M", [1, 8, 16])
def test_pooler_shards(gpu_lib, N, M):
    x, w = synthetic.gemm_inputs(N=N, K=8192, seed=4)
    _say(f"pooler N={N} M={M}")
    _parity_and_repeats(gpu_lib, x, w, M, f"pooler N={N} M={M}")


def test_pooler_weight_ring_layers(gpu_lib):
    """60 distinct W on the device (the pooler ring); layers 0 and 59 checked."""
    import torch

    N, K, M = 512, 8192, 8
    _say("pooler ring 60 layers")
    ring = synthetic.device_weight_ring(60, N, K, "cuda")
    x_bits, _ = synthetic.gemm_inputs(N=16, K=K, seed=5)
    x = to_dev(x_bits[:M])
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in ring]
    for w, y in zip(ring, ys):
        gpu_lib.skinny_gemm_bf16(x, w, y, 0)
    torch.cuda.synchronize()
    for l in (0, 59):
        ref = oracle.gemm_bf16(x_bits[:M], from_dev(ring[l]), THREADS)
        assert_gemm_close(from_dev(ys[l]), ref, f"ring layer {l}")


def _all_launches(sk, M, N, K):
    out = []
    rows_of = {sk.SKINNY_PATH_MFMA: (16, 32, 64), sk.SKINNY_PATH_DOT2: (2, 4, 8, 16),
               sk.SKINNY_PATH_MFMA_4X4: (4, 8)}
    k_of = {sk.SKINNY_PATH_MFMA: 32, sk.SKINNY_PATH_DOT2: 512, sk.SKINNY_PATH_MFMA_4X4: 128}
    for path in rows_of:
        for splits in (1, 2, 4, 8, 16):
            for chunks in (1, 2, 4, 8, 16):
                for accs in (1, 2, 4):
                    mfma = path == sk.SKINNY_PATH_MFMA
                    for rows in rows_of[path]:
                        kw = k_of[path] * chunks
                        waves = (rows // 16 if mfma else 1) * -(-K // (splits * kw))
                        l = sk.Launch(path, splits, waves, chunks, accs, rows)
                        if sk.skinny_launch_unsupported(M, N, K, l) is None:
                            out.append(l)
    return out


@pytest.mark.parametrize("M,N,K", [(1, 64, 1024), (3, 48, 1000), (7, 128, 2048), (16, 32, 520),
                                   (16, 32, 8000)])
def test_every_launch_shape(gpu_lib, M, N, K):
    """Every compiled variant the validator accepts, on a small ragged case
    (N with tiles % 8 != 0, K not a multiple of the chunk)."""
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=6)
    ref = oracle.gemm_bf16(x[:M], w, THREADS)
    launches = _all_launches(gpu_lib, M, N, K)
    assert launches
    for l in launches:
        _say(f"M={M} N={N} K={K} {l}")
        assert_gemm_close(_run(gpu_lib, x, w, M, launch=l), ref, f"{l}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 13, 16])
def test_exact_integer_inputs_bit_exact(gpu_lib, M):
    """Integer inputs whose every partial sum is exact in FP32: each launch
    shape must reproduce the oracle bit for bit."""
    N, K = 256, 2048
    x, w = synthetic.exact_integer_inputs(M=16, N=N, K=K, seed=M)
    ref = oracle.gemm_bf16(x[:M], w, THREADS)
    for l in _all_launches(gpu_lib, M, N, K):
        y = _run(gpu_lib, x, w, M, launch=l, poison=False)
        assert np.array_equal(y, ref), f"{l} not bit-exact at M={M}"


@pytest.mark.parametrize("N,K", [(1024, 4096), (512, 8192), (4096, 8192), (8192, 1024)])
@pytest.mark.parametrize("M", [9, 16])
def test_exact_integer_inputs_at_the_shard_launches(gpu_lib, N, K, M):
    """The chooser's launch on each shard shape, the one the benchmark times
    (at 9..16 tokens the unpooler and pooler shards take token groups, the
    full pooler a walk), reproduces the oracle bit for bit on integer inputs
    whose every partial sum is exact in FP32."""
    x, w = synthetic.exact_integer_inputs(M=16, N=N, K=K, seed=M)
    _say(f"exact integers at the chooser's launch: M={M} N={N} K={K} "
         f"{tuple(gpu_lib.skinny_choose(M, N, K, 0))}")
    assert np.array_equal(_run(gpu_lib, x, w, M), oracle.gemm_bf16(x[:M], w, THREADS))


@pytest.mark.parametrize("M,N,K", [(1, 16, 8), (16, 16, 8), (2, 16, 32), (5, 80, 8), (16, 16, 4104),
                                   (1, 16, 65536), (16, 32, 65536), (4, 65536, 64),
                                   (16, 49152, 520), (12, 2048, 4096), (9, 1024, 8192),
                                   (16, 1040, 6000)])
def test_edge_shapes(gpu_lib, M, N, K):
    """Single rows and tiles, K of one 16-byte piece, long K (split-K with 16
    waves per split), very wide N (16384 workgroups), a wide 16-token MFMA
    call, and shapes outside the table that the chooser's rule gives to the
    16-block MFMA (9-16 tokens, N / 4 >= 256, K 4096..8192, a ragged last
    load group)."""
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=7)
    _say(f"edge M={M} N={N} K={K}")
    assert_gemm_close(_run(gpu_lib, x, w, M), oracle.gemm_bf16(x[:M], w, THREADS), "edge")


@pytest.mark.parametrize("M,N,K", [(4, 16, 524288), (8, 16, 262144), (16, 32, 131072),
                                   (2, 1 << 24, 8)])
def test_size_limits(gpu_lib, M, N, K):
    """The longest K the chooser supports at 4, 8 and 16 tokens (16 splits of
    16 waves, the 16-partial reduction) and the widest N (2^24 features, 8M
    workgroups)."""
    assert gpu_lib.skinny_gemm_unsupported(M, N, K) is None
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=8)
    _say(f"limit M={M} N={N} K={K} {gpu_lib.skinny_choose(M, N, K, 0)}")
    assert_gemm_close(_run(gpu_lib, x, w, M), oracle.gemm_bf16(x[:M], w, THREADS), "limit")


def test_graph_capture_replay(gpu_lib):
    """The GEMM recorded in a HIP graph (allocates nothing, no host sync),
    replayed with new inputs and eager work between replays."""
    import torch

    N, K = 1024, 4096
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=8)
    x2_bits, _ = synthetic.gemm_inputs(N=16, K=K, seed=9)
    for M, splits in ((1, 0), (8, 4), (16, 0)):
        _say(f"graph M={M} S={splits}")
        x = to_dev(x_bits[:M])
        w = to_dev(w_bits)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        gpu_lib.skinny_gemm_bf16(x, w, y, splits)  # warm
        torch.cuda.synchronize()
        eager = from_dev(y).copy()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                gpu_lib.skinny_gemm_bf16(x, w, y, splits)
        torch.cuda.synchronize()
        for rep in range(4):
            y.fill_(7.0)
            src = x_bits if rep % 2 == 0 else x2_bits
            x.copy_(to_dev(src[:M]))
            g.replay()
            torch.cuda.synchronize()
            expect = eager if rep % 2 == 0 else oracle.gemm_bf16(x2_bits[:M], w_bits, THREADS)
            if rep % 2 == 0:
                assert np.array_equal(from_dev(y), expect)
            else:
                assert_gemm_close(from_dev(y), expect, "graph replay with new x")


@pytest.mark.parametrize("path", ["mfma", "mfma_f4", "mfma_4x4", "dot2"])
@pytest.mark.parametrize("splits", [2, 4, 8, 16])
def test_split_k_handoff_alternating_inputs(gpu_lib, path, splits):
    """Back-to-back split calls on alternating weights share the partials
    workspace: a partial left from the previous call would show up as a wrong
    or non-reproducible result."""
    import torch

    N, K, M = 1024, 4096, 4
    if path == "mfma_f4" and splits == 2:
        K = 2048  # 4 tiles x 2 splits cover at most 2048 within 16 waves
    xa, wa = synthetic.gemm_inputs(N=N, K=K, seed=21)
    _, wb = synthetic.gemm_inputs(N=N, K=K, seed=22)
    refs = [oracle.gemm_bf16(xa[:M], wa, THREADS), oracle.gemm_bf16(xa[:M], wb, THREADS)]
    if path == "mfma":
        launch = gpu_lib.Launch(1, splits, -(-K // (splits * 32 * 4)), 4, 2, 16)
    elif path == "mfma_f4":  # 4 tiles a workgroup: the fewest chunks within 16 waves
        chunks = next(c for c in (1, 2, 4, 8, 16) if 4 * -(-K // (splits * 32 * c)) <= 16)
        launch = gpu_lib.Launch(1, splits, 4 * -(-K // (splits * 32 * chunks)), chunks, 2, 64)
    elif path == "mfma_4x4":
        launch = gpu_lib.Launch(3, splits, -(-K // (splits * 128 * 4)), 4, 1, 8)
    else:
        launch = gpu_lib.Launch(0, splits, -(-K // (splits * 512)), 1, 1, 4)
    assert gpu_lib.skinny_launch_unsupported(M, N, K, launch) is None
    _say(f"alternating {path} S={splits} K={K} {launch}")
    x = to_dev(xa[:M])
    ws = [to_dev(wa), to_dev(wb)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(40)]
    for i, y in enumerate(ys):
        gpu_lib.skinny_gemm_bf16_launch(x, ws[i % 2], y, launch)
    torch.cuda.synchronize()
    first = [from_dev(ys[0]), from_dev(ys[1])]
    for j in range(2):
        assert_gemm_close(first[j], refs[j], f"alternating {path} S={splits} weight {j}")
    for i, y in enumerate(ys):
        assert np.array_equal(from_dev(y), first[i % 2]), f"call {i} differs"


@pytest.mark.parametrize("N,K", [(1024, 4096), (8192, 1024), (512, 8192), (4096, 8192),
                                 (2048, 1000), (8192, 3072), (16384, 1024), (2064, 4096),
                                 (2048, 6144), (4096, 4096), (2048, 8192)])
def test_chooser_walk_is_bitwise_the_plain_launch(gpu_lib, N, K):
    """skinny_gemm_bf16 runs some shapes as a persistent walk (the ring kernel
    with one item): bit for bit the plain kernel at skinny_choose's launch,
    within tolerance of the oracle, and no write outside y (the four shard
    shapes, and off-table shapes whose 9-16 token calls run the staged walk,
    one segment a workgroup, up to 4 output blocks a segment, a ragged K, or
    a 16-block walk of 2-block segments, and whose 3-8 token calls run the
    DOT2 walk of 2- or 4-block segments)."""
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=31)
    ref16 = oracle.gemm_bf16(x[:16], w, THREADS)  # rows are independent
    for M in (1, 2, 3, 4, 5, 8, 9, 16):
        walk = gpu_lib.skinny_choose_walk(M, N, K, 0)
        launch = gpu_lib.skinny_choose(M, N, K, 0)
        _say(f"chooser N={N} K={K} M={M} walk={walk}")
        y = _run(gpu_lib, x, w, M)
        assert np.array_equal(y, _run(gpu_lib, x, w, M, launch=launch)), f"M={M} {walk}"
        assert_gemm_close(y, ref16[:M], f"M={M} {walk}")


def test_random_shapes_through_the_choosers(gpu_lib):
    """Seeded random shapes (N a multiple of 16 up to 2048, K a multiple of 8
    up to 9000, M 1..16) through skinny_gemm_bf16 (the chooser's launch and
    walk) and skinny_gemm_bf16_ring (the ring chooser, 1..12 items), against
    the oracle; the plain kernel at skinny_choose's launch bit for bit."""
    import torch

    rng = np.random.default_rng(77)
    for case in range(24):
        M = int(rng.integers(1, 17))
        N = 16 * int(rng.integers(1, 129))
        K = 8 * int(rng.integers(1, 1126))
        count = int(rng.integers(1, 13))
        walk = gpu_lib.skinny_choose_walk(M, N, K, 0)
        ring = gpu_lib.skinny_ring_choose(M, N, K, count)
        _say(f"random case {case}: M={M} N={N} K={K} walk={walk} ring(count={count})={ring}")
        x, w = synthetic.gemm_inputs(N=N, K=K, seed=1000 + case)
        ref = oracle.gemm_bf16(x[:M], w, THREADS)
        y = _run(gpu_lib, x, w, M)
        assert_gemm_close(y, ref, f"case {case}")
        assert np.array_equal(y, _run(gpu_lib, x, w, M, launch=walk.gemm if walk.segment == 0
                                      else gpu_lib.skinny_choose(M, N, K, 0))), f"case {case}"
        xs = [to_dev(synthetic.gemm_inputs(N=16, K=K, seed=2000 + case * 16 + i)[0][:M])
              for i in range(count)]
        ws = [to_dev(w)] + [to_dev(synthetic.gemm_inputs(N=N, K=K, seed=3000 + case * 16 + i)[1])
                            for i in range(1, count)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(count)]
        gpu_lib.skinny_gemm_bf16_ring(xs, ws, ys)
        torch.cuda.synchronize()
        for i in (0, count - 1):
            ref_i = oracle.gemm_bf16(from_dev(xs[i]), from_dev(ws[i]), THREADS)
            assert_gemm_close(from_dev(ys[i]), ref_i, f"case {case} ring item {i}")


@pytest.mark.parametrize("M,N,K,splits", [
    (9, 512, 4096, 0), (16, 768, 8192, 0), (12, 1008, 4096, 0), (16, 1536, 4096, 0),
    (13, 2032, 4096, 0), (10, 512, 6000, 0),
    (16, 512, 8192, 4), (9, 1024, 4096, 2), (12, 2048, 4096, 2), (16, 768, 8192, 8),
    (13, 1024, 6144, 4)])
def test_rule_launches_for_many_tokens(gpu_lib, M, N, K, splits):
    """Off the measured table, 9..16 tokens on K = 4096..8192 take the
    16-block launch: without a split count the rows and token groups the rule
    picks, with one its in-kernel split (8 rows, two token groups up to
    N = 1024). Each against the oracle, and bitwise equal on a second run."""
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=5000 + M + N + K)
    launch = gpu_lib.skinny_choose(M, N, K, splits)
    _say(f"rule launch M={M} N={N} K={K} splits={splits}: {tuple(launch)}")
    assert launch.path == gpu_lib.SKINNY_PATH_MFMA_4X4
    assert launch.splits == max(splits, 1)
    y = _run(gpu_lib, x, w, M, splits=splits)
    assert_gemm_close(y, oracle.gemm_bf16(x[:M], w, THREADS), f"M={M} N={N} K={K} S={splits}")
    assert np.array_equal(_run(gpu_lib, x, w, M, splits=splits, poison=False), y)


def test_blocks_split_in_kernel_equals_the_two_kernel_split(gpu_lib):
    """The 16-block path sums its splits inside the kernel (the last of a
    group's workgroups to finish) when the hand-off counters cover the
    groups (2048), else with the split-reduce kernel; both sum s = 0..S-1
    in order, so output blocks computed either way are equal bit for bit.
    N = 16384 at 4 rows is 4096 groups (two kernels); its first 8192
    columns as their own call are 2048 groups (in-kernel)."""
    import torch

    M, K = 16, 2048
    x_bits, w_bits = synthetic.gemm_inputs(N=16384, K=K, seed=41)
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    for splits in (2, 4):
        launch = gpu_lib.Launch(3, splits, -(-K // (splits * 512)), 4, 1, 4)
        _say(f"16-block split S={splits}: 4096 groups against 2048")
        y_two = torch.empty((M, 16384), dtype=torch.bfloat16, device="cuda")
        y_one = torch.empty((M, 8192), dtype=torch.bfloat16, device="cuda")
        gpu_lib.skinny_gemm_bf16_launch(x, w, y_two, launch)
        gpu_lib.skinny_gemm_bf16_launch(x, w[:8192], y_one, launch)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(y_one), from_dev(y_two)[:, :8192])
        cols = np.arange(0, 16384, 97)
        rows = np.arange(M).repeat(cols.size)
        ref, _ = oracle.gemm_bf16_sampled(x_bits[:M], w_bits, rows, np.tile(cols, M))
        assert_gemm_close(from_dev(y_two)[:, cols].ravel(), ref, f"S={splits} sampled")


@pytest.mark.parametrize("N,K", [(1024, 4096), (512, 8192), (48, 1000)])
def test_token_groups_are_bitwise_one_group(gpu_lib, N, K):
    """The 16-block path's token groups (accs = H: each workgroup takes 4Q of
    the M tokens over all of its K range) compute every token with the same
    instructions in the same order as H = 1, so the outputs are equal bit
    for bit, with and without splits, also when the last group holds fewer
    than 4Q tokens. N = 48 gives 12 or 6 row groups (not a multiple of 8:
    the plain workgroup order), K = 1000 a ragged last chunk."""
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=71)
    n = 0
    for M in (2, 5, 8, 9, 12, 13, 16):
        checked = False
        for rows in (4, 8):
            for chunks in (4, 8):
                for S in (1, 2):
                    one = gpu_lib.Launch(3, S, -(-K // (S * 128 * chunks)), chunks, 1, rows)
                    if gpu_lib.skinny_launch_unsupported(M, N, K, one) is not None:
                        continue
                    y1 = _run(gpu_lib, x_bits, w_bits, M, launch=one)
                    if not checked:
                        assert_gemm_close(y1, oracle.gemm_bf16(x_bits[:M], w_bits, THREADS),
                                          f"M={M} {one}")
                        checked = True
                    for H in (2, 4):
                        l = one._replace(accs=H)
                        if gpu_lib.skinny_launch_unsupported(M, N, K, l) is not None:
                            continue
                        _say(f"token groups M={M} N={N} K={K} {l}")
                        y2 = _run(gpu_lib, x_bits, w_bits, M, launch=l)
                        assert np.array_equal(y2, y1), f"M={M} {l}"
                        n += 1
    assert n >= 20


def test_token_groups_through_the_two_kernel_split(gpu_lib):
    """Token groups multiply the output blocks: N = 8192 at 4 rows is 2048
    blocks at H = 1 (splits summed inside the kernel) and 4096 or 8192 at
    H = 2 or 4, past the 2048 hand-off counters (splits summed by the
    split-reduce kernel). Both add s = 0..S-1 in order: equal bit for bit."""
    M, N, K = 16, 8192, 2048
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=72)
    for S in (2, 4):
        one = gpu_lib.Launch(3, S, -(-K // (S * 512)), 4, 1, 4)
        y1 = _run(gpu_lib, x_bits, w_bits, M, launch=one)
        for H in (2, 4):
            _say(f"token groups H={H} S={S}: two-kernel split against the in-kernel one")
            assert np.array_equal(_run(gpu_lib, x_bits, w_bits, M, launch=one._replace(accs=H)),
                                  y1), f"S={S} H={H}"
        cols = np.arange(0, N, 61)
        rows = np.arange(M).repeat(cols.size)
        ref, _ = oracle.gemm_bf16_sampled(x_bits[:M], w_bits, rows, np.tile(cols, M))
        assert_gemm_close(y1[:, cols].ravel(), ref, f"S={S} sampled")


_RECOMPUTE_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import moe_decode_skinny_amd as sk, synthetic
from tests.helpers import to_dev, from_dev
sk.init(0)
out = {}
for i, (M, N, K, S, H) in enumerate(CASES):
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=50 + i)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    launch = sk.Launch(3, S, -(-K // (S * 512)), 4, H, 4)
    sk.skinny_gemm_bf16_launch(to_dev(x[:M]), to_dev(w), y, launch)
    if S == 2:
        y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        sk.skinny_gemm_bf16(to_dev(x[:M]), to_dev(w), y2, 0)
        torch.cuda.synchronize()
        out[f"chooser{i}"] = from_dev(y2)
    torch.cuda.synchronize()
    out[f"case{i}"] = from_dev(y)
np.savez(sys.argv[2], **out)
print("child done", flush=True)
"""
# (M, N, K, S, token groups H)
_RECOMPUTE_CASES = [(16, 512, 8192, 2, 1), (9, 1024, 4096, 4, 1), (16, 48, 1000, 2, 1),
                    (5, 256, 6000, 8, 1), (16, 512, 8192, 2, 2), (13, 1024, 4096, 4, 4),
                    (9, 48, 1000, 2, 2)]


def test_blocks_split_recompute_path_is_bitwise_the_handoff(gpu_lib, tmp_path):
    """When a group's split workgroups ran on more than one XCD, the last of
    them recomputes every split itself (same instructions, same order)
    instead of reading partials another XCD's L2 holds.  A child process
    with SKINNY_FORCE_SPLIT_RECOMPUTE=1 takes that path on every call; its
    outputs must equal this process's bit for bit."""
    import subprocess

    import torch

    out = tmp_path / "child.npz"
    env = dict(os.environ, SKINNY_FORCE_SPLIT_RECOMPUTE="1")
    code = _RECOMPUTE_CHILD.replace("CASES", repr(_RECOMPUTE_CASES))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    _say("child process with SKINNY_FORCE_SPLIT_RECOMPUTE=1")
    res = subprocess.run([sys.executable, "-c", code, root, str(out)], env=env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    child = np.load(out)
    for i, (M, N, K, S, H) in enumerate(_RECOMPUTE_CASES):
        x, w = synthetic.gemm_inputs(N=N, K=K, seed=50 + i)
        launch = gpu_lib.Launch(3, S, -(-K // (S * 512)), 4, H, 4)
        y = _run(gpu_lib, x, w, M, launch=launch)
        _say(f"recompute case {i}: M={M} N={N} K={K} S={S} H={H}")
        assert np.array_equal(child[f"case{i}"], y), f"case {i}"
        assert_gemm_close(y, oracle.gemm_bf16(x[:M], w, THREADS), f"case {i}")
        if S == 2:
            assert np.array_equal(child[f"chooser{i}"], _run(gpu_lib, x, w, M)), f"chooser {i}"
    torch.cuda.synchronize()


def test_handoff_split_counts_interleaved_on_the_same_blocks(gpu_lib):
    """The in-kernel hand-off's counter word and partial slots of an output
    block are shared by every split count: each call must leave the counter
    at zero and read only partials its own workgroups stored, never those an
    earlier call (another split count, other inputs) left behind.  The
    pooler shard at 16 tokens on 4-row blocks with 2, 4, 8 and 16 splits
    (the same 128 output blocks) and four activation sets, called in
    rotating orders: every output equals its first call's bits and the
    oracle."""
    import torch

    M, N, K = 16, 512, 8192
    _, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=71)
    xs = [synthetic.gemm_inputs(N=16, K=K, seed=72 + j)[0][:M] for j in range(4)]
    w = to_dev(w_bits)
    xd = [to_dev(xb) for xb in xs]
    launches = {S: gpu_lib.Launch(3, S, K // (S * 512), 4, 1, 4) for S in (2, 4, 8, 16)}
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    first = {}
    for rnd in range(3):
        order = [(S, j) for j in range(4) for S in (2, 4, 8, 16)]
        order = order[5 * rnd:] + order[:5 * rnd]
        if rnd == 2:
            order.reverse()
        for S, j in order:
            _say(f"interleaved hand-off round {rnd}: S={S} x{j}")
            y.fill_(7.0)
            gpu_lib.skinny_gemm_bf16_launch(xd[j], w, y, launches[S])
            torch.cuda.synchronize()
            got = from_dev(y).copy()
            if (S, j) not in first:
                assert_gemm_close(got, oracle.gemm_bf16(xs[j], w_bits, THREADS), f"S={S} x{j}")
                first[(S, j)] = got
            else:
                assert np.array_equal(got, first[(S, j)]), f"round {rnd} S={S} x{j}"


def test_in_kernel_split_across_graph_replays(gpu_lib):
    """The pooler shard at 16 tokens in the 16-block launch with 4 splits
    summed inside the kernel; its hand-off counters must be back at zero
    after every call. A captured call replayed with new inputs, eager calls
    of other split launches (one with token groups) on the same workspace
    between replays: every replay equals the eager call bit for bit (same
    x) or the oracle (new x)."""
    import torch

    M, N, K = 16, 512, 8192
    launch = gpu_lib.Launch(3, 4, 4, 4, 1, 4)
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=61)
    x2_bits, _ = synthetic.gemm_inputs(N=16, K=K, seed=62)
    xo, wo = synthetic.gemm_inputs(N=1024, K=4096, seed=63)
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yo = torch.empty((9, 1024), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_gemm_bf16_launch(x, w, y, launch)
    torch.cuda.synchronize()
    eager = from_dev(y).copy()
    assert_gemm_close(eager, oracle.gemm_bf16(x_bits[:M], w_bits, THREADS), "eager")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gpu_lib.skinny_gemm_bf16_launch(x, w, y, launch)
    torch.cuda.synchronize()
    # other in-kernel splits in between: the same blocks' counters, and
    # twice as many output blocks with two token groups
    others = [gpu_lib.Launch(3, 2, 4, 4, 1, 4), gpu_lib.Launch(3, 2, 4, 4, 2, 4)]
    ref2 = oracle.gemm_bf16(x2_bits[:M], w_bits, THREADS)
    for rep in range(6):
        _say(f"in-kernel split graph replay {rep}")
        y.fill_(3.0)
        x.copy_(to_dev((x_bits if rep % 2 == 0 else x2_bits)[:M]))
        gpu_lib.skinny_gemm_bf16_launch(to_dev(xo[:9]), to_dev(wo), yo, others[rep % 2])
        g.replay()
        torch.cuda.synchronize()
        if rep % 2 == 0:
            assert np.array_equal(from_dev(y), eager), f"replay {rep}"
        else:
            assert_gemm_close(from_dev(y), ref2, f"replay {rep}")
