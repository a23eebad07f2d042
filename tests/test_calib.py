"""The MFMA calibration entry point: argument checks and flop count on the CPU (nothing
is launched on an error), a plausible rate and clock on the GPU."""
import pytest

import sigmoid_attention_amd as S


def test_calibrate_rejects_bad_arguments():
    lib = S.load()
    assert lib.sigattn_calibrate_mfma(0, 1, None, None, None) == 1
    assert lib.sigattn_calibrate_mfma(1, 0, None, None, None) == 1
    assert lib.sigattn_calibrate_mfma(1, 1, None, None, None) == 1
    assert lib.sigattn_calibrate_mfma((1 << 16) + 1, 1, 16, 16, None) == 1
    assert lib.sigattn_calibrate_mfma(1, (1 << 20) + 1, 16, 16, None) == 1
    assert lib.sigattn_calibrate_mfma(1 << 16, 1 << 9, 16, 16, None) == 1   # over 2^24 in all
    assert lib.sigattn_calibrate_mfma(1, 1, 18, 16, None) == 3     # sink not 4-byte aligned
    assert lib.sigattn_calibrate_mfma(1, 1, 16, 12, None) == 3     # clk not 8-byte aligned


def test_calibrate_flop_count():
    lib = S.load()
    # workgroups x 4 waves x iterations x 16 MFMAs x (32 x 32 x 16 x 2) flops
    assert lib.sigattn_calibrate_mfma_flops(2, 3) == 2 * 4 * 3 * 16 * 32768
    assert lib.sigattn_calibrate_mfma_flops(0, 3) == 0.0


@pytest.mark.gpu
def test_calibrate_rate_and_clock_are_plausible():
    from gpu_util import need_gpu
    need_gpu()
    r = S.calibrate_mfma(nblocks=1024, iters=1024)
    print(f"\ncalibration: {r['tflops']:.0f} TFLOP/s at {r['sclk_mhz']:.0f} MHz", flush=True)
    # at most the dense bf16 peak at the top clock, and far above any fallback
    assert 300.0 < r["tflops"] < 2600.0
    assert 800.0 < r["sclk_mhz"] < 2600.0
    # the rate matches the clock: 1024 flops per cycle per SIMD, 1024 SIMDs
    assert r["tflops"] < 1.03 * 1024 * 1024 * r["sclk_mhz"] * 1e6 / 1e12
