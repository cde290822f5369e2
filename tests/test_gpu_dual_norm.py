"""GPU parity of the single-GPU dual norm (skinny_dual_norm) through the C ABI,
against the oracle's reading of it (oproj.batt page, AttentionBoundary:
post_attn_norm, gated add into the FP32 residual stream in place,
pre_ffn_norm into BF16; the formula is a reading, see the oracle source).

Both sides compute in binary64 with one rounding per narrowing; only the
order of the two sums of squares differs, which can move a reciprocal root by
an ulp of binary64 and a rounded result only when the exact value lies within
about 2^-53 (relative) of a bfloat16 or binary32 midpoint.  The test asks
for the output and the updated residual bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests.helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(M, H, seed, post=True, alpha_vec=True):
    rng = np.random.default_rng(seed)
    bf = synthetic.to_bf16_bits
    partial = bf(rng.normal(size=(M, H)))
    residual = (2.0 * rng.normal(size=(M, H))).astype(np.float32)
    post_w = bf(rng.normal(0.0, 0.3, H)) if post else None
    alpha = bf(1.0 + rng.normal(0.0, 0.1, H)) if alpha_vec else 0.875
    beta = bf(0.5 + rng.normal(0.0, 0.1, H))
    next_w = bf(rng.normal(0.0, 0.3, H))
    return partial, residual, post_w, alpha, beta, next_w


def _run(sk, partial, residual, post_w, alpha, beta, next_w, consts):
    import torch

    M, H = partial.shape
    p = to_dev(partial)
    r = torch.from_numpy(residual.copy()).cuda()
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    al = alpha if np.isscalar(alpha) else to_dev(alpha)
    sk.skinny_dual_norm(p, r, None if post_w is None else to_dev(post_w), consts[0], consts[1],
                        al, to_dev(beta), to_dev(next_w), consts[2], consts[3], out)
    torch.cuda.synchronize()
    return from_dev(out), r.cpu().numpy()


def _compare(out, res, want_out, want_res, tag):
    bad_out = np.count_nonzero(out != want_out)
    bad_res = np.count_nonzero(res.view(np.uint32) != want_res.view(np.uint32))
    _say(f"{tag}: out differs at {bad_out}, residual at {bad_res} of {out.size}")
    assert np.all(np.isfinite(res)), tag
    assert bad_out == 0 and bad_res == 0, tag


CONSTS = (1.0, 1e-6, 1.0, 1e-6)  # post gain center, post eps, pre gain center, pre eps


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("post,alpha_vec", [(True, True), (False, False), (True, False)])
def test_dual_norm_oproj_rows(gpu_lib, M, post, alpha_vec):
    """The o_proj output width H = 8192."""
    H = 8192
    args = _inputs(M, H, seed=M, post=post, alpha_vec=alpha_vec)
    out, res = _run(gpu_lib, *args, CONSTS)
    want_out, want_res, _ = oracle.dual_norm(args[0], args[1], args[2], CONSTS[0], CONSTS[1],
                                             args[3], args[4], args[5], CONSTS[2], CONSTS[3])
    _compare(out, res, want_out, want_res, f"M={M} post={post} alpha_vec={alpha_vec}")


@pytest.mark.parametrize("M,H", [(3, 16), (2, 48), (5, 4096), (4, 8208), (65, 512)])
def test_dual_norm_shapes(gpu_lib, M, H):
    """One block per row, fewer blocks than threads, several blocks per
    thread with a ragged last round, many rows."""
    args = _inputs(M, H, seed=H)
    consts = (0.5, 1e-5, 1.0, 1e-3)
    out, res = _run(gpu_lib, *args, consts)
    want_out, want_res, _ = oracle.dual_norm(args[0], args[1], args[2], consts[0], consts[1],
                                             args[3], args[4], args[5], consts[2], consts[3])
    _compare(out, res, want_out, want_res, f"M={M} H={H}")


def test_dual_norm_on_the_gemm_output(gpu_lib):
    """The o_proj shard GEMM (M=8, N=8192, K=1024) feeding the dual norm on
    the device; the oracle gets the GPU's GEMM output as its partial."""
    import torch

    M, N, K = 8, 8192, 1024
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=50)
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_gemm_bf16(x, w, y, 0)
    _, residual, post_w, alpha, beta, next_w = _inputs(M, N, seed=51)
    r = torch.from_numpy(residual.copy()).cuda()
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_dual_norm(y, r, to_dev(post_w), 1.0, 1e-6, to_dev(alpha), to_dev(beta),
                             to_dev(next_w), 1.0, 1e-6, out)
    torch.cuda.synchronize()
    want_out, want_res, _ = oracle.dual_norm(from_dev(y), residual, post_w, 1.0, 1e-6, alpha,
                                             beta, next_w, 1.0, 1e-6)
    _compare(from_dev(out), r.cpu().numpy(), want_out, want_res, "gemm -> dual norm")


def test_dual_norm_in_place_across_graph_replays(gpu_lib):
    """The residual is updated in place: a captured call replayed three times
    must match the oracle applied three times, and repeat bit for bit."""
    import torch

    M, H = 4, 8192
    partial, residual, post_w, alpha, beta, next_w = _inputs(M, H, seed=60)
    p, pw, al, be, nw = (to_dev(v) for v in (partial, post_w, alpha, beta, next_w))
    r = torch.from_numpy(residual.copy()).cuda()
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    gpu_lib.skinny_dual_norm(p, r, pw, 1.0, 1e-6, al, be, nw, 1.0, 1e-6, out)  # warm
    torch.cuda.synchronize()
    r.copy_(torch.from_numpy(residual))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gpu_lib.skinny_dual_norm(p, r, pw, 1.0, 1e-6, al, be, nw, 1.0, 1e-6, out)
    torch.cuda.synchronize()
    want_res = residual
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        want_out, want_res, _ = oracle.dual_norm(partial, want_res, post_w, 1.0, 1e-6, alpha,
                                                 beta, next_w, 1.0, 1e-6)
        got = r.cpu().numpy()
        _compare(from_dev(out), got, want_out, want_res, f"replay {rep}")
