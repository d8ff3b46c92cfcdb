"""The benchmark's machine probes run and report plausible figures: the bf16
MFMA loop below the vendor's 2.5 PFLOP/s dense peak, the shader clock within
the part's range, the device copy below the 8 TB/s HBM peak."""
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
