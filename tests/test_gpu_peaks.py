"""Matrix-core peaks of the device: the rates derived from its CU count and
clock (what the published MI355X figures are made of: 256 CUs at 2.4 GHz,
256 / 128 / 4096 / 8192 dense MFMA flops (int8: operations) per clock per CU
for float32 / float64 / fp16 / int8) and the rates register-only MFMA loops
reach through the library."""

import pytest

from matrix_roots_amd import binding as B

pytestmark = pytest.mark.gpu

VENDOR = {"f32": 157.3, "f64": 78.6, "f16": 2500.0, "i8": 5000.0}


def test_measure_peaks(gpu_available):
    p = B.measure_peaks()
    print(p)
    assert p["cu_count"] > 0 and p["clock_mhz"] > 0
    for k, v in VENDOR.items():
        prop = p["device_prop_tflops"][k]
        meas = p["measured_tflops"][k]
        # the derived figure is the vendor's own arithmetic on this device
        assert 0.8 * v <= prop <= 1.2 * v, (k, prop)
        # a loop without memory traffic reaches most of it and cannot beat it
        assert 0.5 * prop <= meas <= 1.05 * prop, (k, meas, prop)
        # random operands: the clock the chip holds with real data (lower for
        # int8 and fp16; float32 and float64 draw about the same either way)
        rnd = p["measured_random_tflops"][k]
        assert 0.3 * prop <= rnd <= 1.05 * prop, (k, rnd, prop)
