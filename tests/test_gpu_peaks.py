"""GPU: the achievable-rate probes of libsa_peaks.so (measurement only) launch,
report the work they did, and give rates in a sane range on an MI355X: the
bf16 product loops (one operand pair; changing data) below the 2.5 PFLOP/s
datasheet figure, the LDS reads near
or below 256 bytes a clock per CU at 2.4 GHz, the streaming read finite (a
512 MiB buffer partly hits the 256 MB last-level cache).  Short runs: the
rates are checked for plausibility, not measured."""

import math

import pytest

import bench
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def test_peak_probes_report_plausible_rates():
    import torch
    dev = torch.device("cuda", 0)
    say("peaks probes: read 512 MiB, 2000 product rounds, 2000 LDS rounds")
    hbm, mfma, mfma_data, lds = bench.achievable_peaks(dev, read_mib=512, reps=2, mfma_iters=2000,
                                                        lds_iters=2000)
    say(f"  HBM {hbm:.0f} GB/s, MFMA {mfma:.0f} / {mfma_data:.0f} TFLOP/s (one pair / changing data), "
        f"LDS {lds:.0f} GB/s per CU")
    for x in (hbm, mfma, mfma_data, lds):
        assert math.isfinite(x) and x > 0.0
    # upper bounds from the datasheet (a 512 MiB buffer may partly hit the
    # last-level cache, so only the product and LDS rates get lower bounds)
    assert mfma < 2500.0 and mfma > 500.0
    assert mfma_data < 2500.0 and mfma_data > 500.0
    assert lds < 1.1 * 256 * 2.4 and lds > 100.0
    assert hbm < 20000.0
