"""GPU parity for the fused launch of several matrices (lutq_matmul_multi).

- each output against the oracle, for every path and workgroup shape, with
  and without K splits, grouped and tensor-wise scales, ragged widths and
  ragged / sliced batches;
- each output bit-identical to the single-matrix launch with the same path,
  shape and split (workgroups never span two matrices);
- the Llama-3-8B layer's q/k/v and gate/up at the benchmark's batch sizes,
  every output compared, under the automatic plan;
- degenerate cases: one matrix, an empty matrix among others, K = 0.
"""

import numpy as np
import pytest

import oracle
from synth import draw, tables, workloads

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


def make_mats(bits, table, group, widths, K, seed):
    """Per matrix: codes, its own table (a permutation of one kind) and scales."""
    out = []
    for i, N in enumerate(widths):
        c, T, s, _ = workloads.small_case(bits, table, group, 1, N, K, seed=seed + 17 * i)
        perm = np.random.default_rng(seed + i).permutation(1 << bits)
        out.append((c, T[perm], s))          # a different table per matrix
    return out


def upload(lutq, mats, bits, group):
    return [(lutq.repack(dev(c), bits, group), dev(T), dev(s)) for c, T, s in mats]


def check(ys, x, mats, group):
    for y, (c, T, s) in zip(ys, mats):
        y_ref, B = oracle.reference(x, c, T, s, group)
        ok, worst = oracle.check(y.cpu().numpy(), y_ref, B)
        assert ok, f"max err/bound = {worst:.3g}"


SHAPES = [("gemv", 1), ("gemv", 2), ("mfma", 1), ("mfma", 2), ("mfma", 4), ("mfma", 7), ("mfma", 8)]


@pytest.mark.parametrize("path,tiles", SHAPES)
@pytest.mark.parametrize("bits,table,group", [(4, "nf", 128), (3, "lloyd_max", 0), (2, "int", 256)])
@pytest.mark.parametrize("M", [1, 5, 16, 45])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_fused_matches_oracle_and_single(lutq, path, tiles, bits, table, group, M, ksplit):
    # widths: 19 tiles (ragged last tile), 4 tiles, 1 partial tile, 9 tiles
    widths, K = [293, 64, 5, 140], 768
    mats = make_mats(bits, table, group, widths, K, seed=500 + bits + M)
    x = draw.activations(M, K, (501, M))
    dm = upload(lutq, mats, bits, group)
    xd = dev(x)
    ys = lutq.matmul_multi(xd, dm, path=path, tiles=tiles, ksplit=ksplit)
    torch.cuda.synchronize()
    check(ys, x, mats, group)
    for y, (P, T, s) in zip(ys, dm):
        y1 = lutq.matmul(xd, P, T, s, path=path, tiles=tiles, ksplit=ksplit)
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


# gate + up: 1792 tiles, 7 per wave (one workgroup per CU) from 2 batch rows
@pytest.mark.parametrize("names,Ms", [(("q", "k", "v"), (1, 8, 16, 32)), (("gate", "up"), (1, 8, 16, 32))])
def test_fused_llama_layer(lutq, names, Ms):
    w = workloads.WORKLOADS["nf4_layer"]
    mats, dm = [], []
    for n in names:
        c, T, s = workloads.quantized(w, n)
        mats.append((c, T, s))
        dm.append((lutq.repack(dev(c), w.bits, w.group), dev(T), dev(s)))
    for M in Ms:
        x = workloads.activations(w, M, names[0])
        ys = lutq.matmul_multi(dev(x), dm)
        torch.cuda.synchronize()
        for y, (c, T, s) in zip(ys, mats):
            # every output of every matrix
            y_ref, B = oracle.reference(x, c, T, s, w.group)
            ok, worst = oracle.check(y.cpu().numpy(), y_ref, B)
            assert ok, f"{M=} max err/bound = {worst:.3g}"


def test_fused_degenerate(lutq):
    K = 256
    mats = make_mats(4, "nf", 128, [70, 33], K, seed=510)
    dm = upload(lutq, mats, 4, 128)
    x = draw.activations(3, K, (511,))
    xd = dev(x)
    # one matrix
    (y,) = lutq.matmul_multi(xd, dm[:1])
    check([y], x, mats[:1], 128)
    # an empty matrix among others is skipped
    c0 = np.zeros((0, K), np.uint8)
    P0 = lutq.repack(torch.empty((0, K), dtype=torch.uint8, device="cuda"), 4, 128)
    e = (P0, dm[0][1], torch.empty((0, 2), dtype=torch.float16, device="cuda"))
    ys = lutq.matmul_multi(xd, [dm[0], e, dm[1]])
    assert ys[1].shape == (3, 0)
    check([ys[0], ys[2]], x, mats, 128)
    # K = 0: every output is zero
    Pk = [lutq.repack(torch.empty((n, 0), dtype=torch.uint8, device="cuda"), 4, 0) for n in (20, 7)]
    lut = dm[0][1]
    sc = torch.ones(1, dtype=torch.float16, device="cuda")
    outs = [torch.full((2, n), 1.0, dtype=torch.float16, device="cuda") for n in (20, 7)]
    ys = lutq.matmul_multi(torch.empty((2, 0), dtype=torch.float16, device="cuda"),
                           [(Pk[0], lut, sc), (Pk[1], lut, sc)], outs=outs)
    torch.cuda.synchronize()
    assert all(bool((y == 0).all()) for y in ys)
    # mismatched K is rejected (by the binding; the C entry point's own check is
    # covered on the CPU in test_abi.py)
    Pbad = lutq.repack(dev(mats[0][0][:, :128]), 4, 128)
    with pytest.raises(ValueError):
        lutq.matmul_multi(xd, [dm[0], (Pbad, dm[0][1], dm[0][2])])
