"""mifa_clock_probe on the GPU: every probe runs for its span of real time and reports an engine
clock within the chip's range."""
import pytest

torch = pytest.importorskip("torch")


@pytest.mark.gpu
def test_clock_probe_reports_a_plausible_clock():
    from io_aware_softmax_mifa_amd import binding

    print("clock probe: span 20 ms, 8 probes", flush=True)
    buf = torch.zeros(32, dtype=torch.int64, device="cuda")
    st, khz = binding.mifa_clock_probe_raw(buf, 20_000, torch.cuda.current_stream().cuda_stream)
    assert st == 0 and khz > 0
    torch.cuda.synchronize()
    v = buf.cpu().tolist()
    for w in range(8):
        t0, r0, t1, r1 = v[4 * w:4 * w + 4]
        assert r1 - r0 >= 20_000 * khz // 1000  # the whole span of real time passed
        assert r1 - r0 < 1_000_000 * khz // 1000  # and ended well within a second
        mhz = (t1 - t0) / (r1 - r0) * khz / 1e3
        assert 100.0 < mhz < 3000.0, (w, mhz)
