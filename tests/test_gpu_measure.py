"""The measurement helpers of libqgemm on the GPU: they run, and the device
figures they derive the ceilings from are those of one MI355X."""
import pytest

torch = pytest.importorskip("torch")
import bit_weight_only_dequant_amd as qgm  # noqa: E402

pytestmark = pytest.mark.gpu


def test_device_info_is_an_mi355x():
    info = qgm.device_info(0)
    assert info["compute_units"] == 256
    assert 1_000_000 <= info["clock_khz"] <= 3_000_000
    assert info["memory_bus_bits"] > 0


def test_stream_read_and_empty_launch_run():
    buf = torch.ones(6684672 // 2 + 8, dtype=torch.float16, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    for wg in (256, 2048):
        qgm.stream_read(buf, 6684672 + 3, sink, wg)   # a ragged tail of 3 bytes
    qgm.empty_launch(768, 512)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0   # the fold of all-ones data never equals the sentinel


def test_mfma_probe_runs_and_rejects_a_small_output():
    out = torch.empty(8 * 256, dtype=torch.float32, device="cuda")
    qgm.mfma_probe(out, 8, 3)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    with pytest.raises(ValueError):
        qgm.mfma_probe(out, 9, 3)


def test_clock_stamps_bracket_the_launches_between_them():
    # two stamps in a graph around launches of known duration: the span grows
    # with the work between them, and agrees with events around a long run
    khz = qgm.clock_rate_khz(0)
    assert 1_000 <= khz <= 10_000_000
    out = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
    ts = torch.zeros(2, dtype=torch.int64, device="cuda")
    spans = []
    for iters in (200, 2000):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qgm.clock_stamp(ts[0:1])
            qgm.mfma_probe(out, 64, iters)
            qgm.clock_stamp(ts[1:2])
        for _ in range(2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
        t = ts.cpu().tolist()
        span_ms = (t[1] - t[0]) / khz
        assert 0.0 < span_ms <= a.elapsed_time(b) * 1.05 + 0.02
        spans.append(span_ms)
    assert spans[1] > 5.0 * spans[0]   # ten times the MFMA rounds between the stamps
    with pytest.raises(ValueError):
        qgm.clock_stamp(torch.zeros(2, dtype=torch.int32, device="cuda"))
