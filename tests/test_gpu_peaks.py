"""The peak microbenchmarks (include/lutq_peaks.h) launch and complete on the
GPU for every kind and size bench.py uses, and a stream with a store writes
its sink (the XOR of the bytes each wave read, here of zeros)."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lutq():
    import weight_only_lut_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def test_peaks_launch_and_complete(lutq):
    lutq.peak_empty()
    buf = torch.zeros(4 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((lutq.peak_stream_sink_bytes(),), 0xAB, dtype=torch.uint8, device="cuda")
    for store in (False, True):
        lutq.peak_stream(buf, 4 << 20, store, sink)
    torch.cuda.synchronize()
    assert int(sink.max().item()) == 0           # every wave's four stores landed (zeros read)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fsink = torch.zeros(cus * 16, dtype=torch.float32, device="cuda")
    for kind in (lutq.PEAK_MFMA_16X16X32, lutq.PEAK_MFMA_32X32X16):
        for wps in (1, 2, 4):
            lutq.peak_mfma(kind, wps, 3, fsink)
    isink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for wpc in (4, 8, 16):
        lutq.peak_lds(wpc, 3, isink)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(fsink).all())
