"""lutq_matmul_noalloc: the split-K product with its scratch in the library's
fixed per-GPU array. Called through the C ABI, it gives lutq_matmul_ex's
bits for the same options, on two calls in a row (the second smaller), in a
graph captured on a stream that has no scratch of its own, and it refuses a
split larger than the array with nothing enqueued."""

import numpy as np
import pytest

from synth import draw, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lutq():
    import weight_only_lut_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(lutq, N, K, M, seed, bits=4, table="nf"):
    c, T, s, _ = workloads.small_case(bits, table, 128, 1, N, K, seed=seed)
    P = lutq.repack(dev(c), bits, 128)
    return P, dev(T), dev(s), dev(draw.activations(M, K, (seed, 1)))


@pytest.mark.parametrize("path,ksplit,tiles,M", [("gemv", 4, 2, 8), ("mfma", 3, 2, 32),
                                                  ("mfma", 2, 4, 20), ("auto", 0, 0, 16)])
def test_noalloc_equals_matmul_ex_twice(lutq, path, ksplit, tiles, M):
    kw = dict(path=path, ksplit=ksplit, tiles=tiles)
    # first call, then a smaller one: each bit-identical to lutq_matmul_ex
    for N, K, m, seed in ((700, 2048, M, 990), (90, 1024, max(1, M // 3), 991)):
        P, T, s, x = case(lutq, N, K, m, seed)
        want = lutq.matmul(x, P, T, s, **kw)
        got = lutq.matmul_noalloc(x, P, T, s, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (N, K, m)


def test_noalloc_under_capture_on_a_fresh_stream(lutq):
    P, T, s, x = case(lutq, 300, 1024, 8, 992, bits=3, table="lloyd_max")
    want = lutq.matmul(x, P, T, s, path="gemv", ksplit=4)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()   # lutq_matmul_ex would need to allocate here
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        out = lutq.matmul_noalloc(x, P, T, s, path="gemv", ksplit=4)
    for rep in range(3):
        with torch.cuda.stream(stream):
            out.view(torch.int16).fill_(0x7E00)
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep


def test_noalloc_refuses_splits_beyond_its_array(lutq):
    # 128 row blocks x 16 splits x 32 rows x 32 batch rows of fp32 = 8 MiB,
    # more than the array holds after its 64 KiB of counters
    P, T, s, x = case(lutq, 4096, 2048, 32, 993)
    y = torch.full((32, 4096), 3.0, dtype=torch.float16, device="cuda")
    with pytest.raises(lutq.LutqError) as e:
        lutq.matmul_noalloc(x, P, T, s, path="mfma", tiles=2, ksplit=16, out=y)
    assert e.value.code == -8
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # one split fewer fits, and matches lutq_matmul_ex
    want = lutq.matmul(x, P, T, s, path="mfma", tiles=2, ksplit=15)
    got = lutq.matmul_noalloc(x, P, T, s, path="mfma", tiles=2, ksplit=15)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
