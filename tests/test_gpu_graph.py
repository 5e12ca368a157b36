"""HIP graphs and streams: the launches captured in a graph and replayed
several times (with eager work and synchronisation between replays) give
every time the eager results bit for bit, for the plain, split-K, fused,
zero-point, bf16 and binary-coded paths; split-K launches on two streams at
once (each stream has its own scratch) give their single-stream results.

A split-K launch allocates its scratch on first use, so each case runs once
eagerly before capture, as the benchmark does. A capture that would need new
scratch is refused (LUTQ_ECAPTURE) with nothing enqueued, and a graph keeps
working after a later eager call on its stream has outgrown the scratch it
was captured with (the outgrown buffer is retired, not freed).
"""

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


def bits16(t):
    return t.view(torch.int16).clone()


def _cases(lutq):
    K = 1024
    c, T, s, _ = workloads.small_case(4, "nf", 128, 1, 300, K, seed=950)
    P = lutq.repack(dev(c), 4, 128)
    Td, sd = dev(T), dev(s)
    z = dev(np.random.default_rng(951).uniform(-0.5, 0.5, s.shape).astype(np.float16))
    c2, T2, s2, _ = workloads.small_case(4, "nf", 128, 1, 64, K, seed=952)
    P2 = lutq.repack(dev(c2), 4, 128)
    T2d, s2d = dev(T2), dev(s2)
    a = np.random.default_rng(953).uniform(0.01, 0.03, (3, 300, K // 128)).astype(np.float16)
    cb = np.random.default_rng(954).integers(0, 8, (300, K)).astype(np.uint8)
    Pb = lutq.repack(dev(cb), 3, 128)
    x8 = dev(draw.activations(8, K, (955,)))
    x32 = dev(draw.activations(32, K, (956,)))
    xb = x8.to(torch.bfloat16)
    ad = dev(a)
    return [
        ("gemv", lambda: lutq.matmul(x8, P, Td, sd, path="gemv")),
        ("gemv split-K", lambda: lutq.matmul(x8, P, Td, sd, path="gemv", ksplit=4)),
        ("mfma split-K", lambda: lutq.matmul(x32, P, Td, sd, path="mfma", ksplit=3)),
        ("fused", lambda: lutq.matmul_multi(x8, [(P, Td, sd), (P2, T2d, s2d)], ksplit=2)),
        ("zero points", lambda: lutq.matmul(x32, P, Td, sd, zeros=z, ksplit=2)),
        ("bf16", lambda: lutq.matmul(xb, P, Td, sd, path="mfma", ksplit=2)),
        ("bcq", lambda: lutq.matmul_bcq(x8, Pb, ad, ksplit=2)),
    ]


def test_graph_replays_equal_eager(lutq):
    cases = _cases(lutq)
    stream = torch.cuda.Stream()
    eager, outs = {}, {}
    with torch.cuda.stream(stream):
        for name, f in cases:
            r = f()
            eager[name] = [bits16(t) for t in (r if isinstance(r, list) else [r])]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for name, f in cases:
            r = f()
            outs[name] = r if isinstance(r, list) else [r]
    for rep in range(4):
        with torch.cuda.stream(stream):
            # poison the outputs, on the replay's stream: the side stream does
            # not wait for work queued on the default one
            for name in outs:
                for t in outs[name]:
                    t.view(torch.int16).fill_(0x7E00)
            graph.replay()
        torch.cuda.synchronize()
        for name in outs:
            for got, want in zip(outs[name], eager[name]):
                assert torch.equal(got.view(torch.int16), want), f"{name}, replay {rep}"
        with torch.cuda.stream(stream):                 # eager work between replays
            cases[1][1]()
        torch.cuda.synchronize()


def test_split_k_on_two_streams_at_once(lutq):
    c, T, s, _ = workloads.small_case(4, "nf", 128, 1, 500, 2048, seed=960)
    P = lutq.repack(dev(c), 4, 128)
    Td, sd = dev(T), dev(s)
    xs = [dev(draw.activations(8, 2048, (961, i))) for i in range(2)]
    want = [bits16(lutq.matmul(x, P, Td, sd, path="gemv", ksplit=5)) for x in xs]
    streams = [torch.cuda.Stream() for _ in range(2)]
    for _ in range(3):
        ys = []
        for st, x in zip(streams, xs):
            with torch.cuda.stream(st):
                ys.append([lutq.matmul(x, P, Td, sd, path="gemv", ksplit=5) for _ in range(10)])
        torch.cuda.synchronize()
        for got_list, w in zip(ys, want):
            for got in got_list:
                assert torch.equal(got.view(torch.int16), w)


def test_graph_survives_scratch_growth(lutq):
    K = 1024
    c, T, s, _ = workloads.small_case(4, "nf", 128, 1, 200, K, seed=970)
    P = lutq.repack(dev(c), 4, 128)
    Td, sd = dev(T), dev(s)
    x = dev(draw.activations(32, K, (971,)))
    # a large split: 256 row blocks x 16 splits x 32 rows x 32 batch rows of
    # fp32 partials is 16 MiB, more than the stream's first buffer holds
    Kb = 2048
    cb, Tb, sb, _ = workloads.small_case(4, "nf", 128, 1, 8192, Kb, seed=972)
    Pb = lutq.repack(dev(cb), 4, 128)
    Tbd, sbd = dev(Tb), dev(sb)
    xb = dev(draw.activations(32, Kb, (973,)))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        want = bits16(lutq.matmul(x, P, Td, sd, path="mfma", tiles=2, ksplit=3))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        out = lutq.matmul(x, P, Td, sd, path="mfma", tiles=2, ksplit=3)
    for rep in range(3):
        with torch.cuda.stream(stream):
            big = lutq.matmul(xb, Pb, Tbd, sbd, path="mfma", tiles=2, ksplit=16)  # grows the scratch
            out.view(torch.int16).fill_(0x7E00)
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want), f"replay {rep}"
    # the growing call itself is right as well (against its unsplit launch)
    ref = lutq.matmul(xb, Pb, Tbd, sbd, path="mfma", tiles=2, ksplit=1).float()
    torch.cuda.synchronize()
    assert torch.allclose(big.float(), ref, rtol=2e-3, atol=1e-4)


def test_capture_refuses_new_scratch(lutq):
    c, T, s, _ = workloads.small_case(4, "nf", 128, 1, 64, 512, seed=980)
    P = lutq.repack(dev(c), 4, 128)
    Td, sd = dev(T), dev(s)
    x = dev(draw.activations(4, 512, (981,)))
    y = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    other = torch.zeros(16, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()   # a stream with no scratch yet
    graph = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(graph, stream=stream):
        try:
            lutq.matmul(x, P, Td, sd, path="gemv", ksplit=2, out=y)
        except lutq.LutqError as e:
            err = e
        other.add_(1.0)
    assert err is not None and err.code == -9, err
    graph.replay()                 # the refused call enqueued nothing
    torch.cuda.synchronize()
    assert int(y.abs().max().item()) == 0 and float(other[0].item()) == 1.0
    with torch.cuda.stream(stream):  # eagerly it runs, and a capture after it works
        want = bits16(lutq.matmul(x, P, Td, sd, path="gemv", ksplit=2))
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=stream):
        out = lutq.matmul(x, P, Td, sd, path="gemv", ksplit=2)
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want)
