"""The matrix-core ceiling probe runs and reports a plausible clock: every
block records a positive cycle and constant-clock count, and the rate stays
below the published dense peaks (bf16 2.5, fp8 5.0 PFLOP/s at 2.4 GHz)."""
import pytest

from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,peak", [("bf16", 2500.0), ("fp8", 5000.0)])
def test_mfma_ceiling_probe(gpu, dtype, peak):
    from whisper_attention_amd import diag
    announce(f"mfma ceiling probe {dtype}")
    r = diag.mfma_ceiling(dtype, iters=256, reps=3)
    print(r, flush=True)
    assert r["wall_clock_kHz"] > 0
    assert r["sclk_MHz"] is not None and 100.0 < r["sclk_MHz"] < 3000.0
    assert 0.0 < r["TFLOP/s"] <= 1.05 * peak * r["sclk_MHz"] / 2400.0


def test_sclk_probe(gpu):
    """The clock probe reads a plausible shader clock and ends on its own."""
    from whisper_attention_amd import diag
    p = diag.SclkProbe(n_blocks=8, spin=200)
    for _ in range(3):
        p.launch()
    mhz = p.mhz()
    assert mhz is not None and 100.0 < mhz < 3000.0
