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
