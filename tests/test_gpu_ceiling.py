"""The benchmark's measurement reference kernels (libskinny_ceiling,
include/skinny_ceiling.h): the stream references read exactly the bytes
their layout says, once, and the stream-and-store reference stores the
documented XOR of them."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PATTERN = 0x5EC0DE42


@pytest.mark.parametrize("L", [1, 2, 4, 8])
def test_stream_reference_reads_its_layout(L):
    """Two threads get data whose XOR is the sink pattern; the sink words of
    exactly the workgroups that hold such a thread (by the documented layout:
    load i of thread t of workgroup b at b*8192L + 8192i + 16t) are set."""
    import torch

    from moe_decode_skinny_amd import ceiling

    print(f"ceiling stream L={L}", flush=True)
    nwg = 6
    rng = np.random.default_rng(70 + L)
    data = rng.integers(0, 2 ** 32, 2048 * L * nwg, dtype=np.uint64).astype(np.uint32)
    view = data.reshape(nwg, L, 512, 4)  # [b][i][t][j]: word b*2048L + 2048i + 4t + j
    for b, t in ((2, 37), (5, 500)):
        x = np.bitwise_xor.reduce(view[b, :, t, :].ravel())
        view[b, 0, t, 0] ^= x ^ np.uint32(PATTERN)
    hit = (np.bitwise_xor.reduce(np.bitwise_xor.reduce(view, axis=3), axis=1) == PATTERN)
    expected = np.where(hit.any(axis=1), 1, 7).astype(np.int32)
    assert list(expected) == [7, 7, 1, 7, 7, 1]
    src = torch.from_numpy(data.view(np.int32)).to("cuda")
    sink = torch.full((nwg,), 7, dtype=torch.int32, device="cuda")
    ceiling.skinny_ceiling_stream(src, sink, L)
    ceiling.skinny_ceiling_empty(0)
    torch.cuda.synchronize()
    assert np.array_equal(sink.cpu().numpy(), expected)


@pytest.mark.parametrize("L", [1, 2, 4, 8])
def test_stream_store_reference_stores_its_xor(L):
    """out[b * 64 + l] is the XOR of every word threads 64 w + l (w < 8) of
    workgroup b read, by the documented layout."""
    import torch

    from moe_decode_skinny_amd import ceiling

    print(f"ceiling stream-and-store L={L}", flush=True)
    nwg = 5
    rng = np.random.default_rng(90 + L)
    data = rng.integers(0, 2 ** 32, 2048 * L * nwg, dtype=np.uint64).astype(np.uint32)
    view = data.reshape(nwg, L, 8, 64, 4)  # [b][i][wave][lane][j]
    want = np.bitwise_xor.reduce(view.transpose(0, 3, 1, 2, 4).reshape(nwg, 64, -1), axis=2)
    src = torch.from_numpy(data.view(np.int32)).to("cuda")
    out = torch.full((nwg * 64,), 7, dtype=torch.int32, device="cuda")
    ceiling.skinny_ceiling_stream_store(src, out, L)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.ravel())
