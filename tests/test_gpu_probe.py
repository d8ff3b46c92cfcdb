"""The benchmark's machine probes run and report plausible figures: the bf16
MFMA loop below the vendor's 2.5 PFLOP/s dense peak, the shader clock within
the part's range, the device copy below the 8 TB/s HBM peak; the benchmark's
fence-less timing events agree with torch's default events."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_measured_peaks_are_plausible():
    import bench
    dev = torch.device("cuda:0")
    mp = bench.measured_peaks(torch, dev, torch.cuda.current_stream(dev))
    assert mp is not None
    print(mp, flush=True)
    assert 200.0 < mp["mfma_bf16_TFs"] < 2600.0
    assert 500.0 < mp["sclk_MHz"] < 3000.0
    assert 500.0 < mp["hbm_copy_GBs"] < 8000.0


def test_timing_events_agree_with_default_events():
    import bench
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = bench.probe_lib()
    cyc = torch.zeros(1, dtype=torch.int64, device=dev)

    def spin():  # one wave spinning 10M shader-clock cycles (some milliseconds)
        assert lib.dnp_clock(10_000_000, ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0

    spin()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0, p1 = bench.TimingEvent(), bench.TimingEvent()
    t0.record(stream)
    p0.record(stream)
    spin()
    p1.record(stream)
    t1.record(stream)
    t1.synchronize()
    ms_t, ms_p = t0.elapsed_time(t1), p0.elapsed_time(p1)
    print("default %.4f ms, fence-less %.4f ms" % (ms_t, ms_p), flush=True)
    assert ms_p > 0.5
    assert abs(ms_t - ms_p) < 0.02 * ms_t + 0.05
