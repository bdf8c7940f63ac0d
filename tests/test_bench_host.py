"""Host-side pieces of bench.py: the gfx clock reading that sits beside the roofline."""
import bench


def test_read_sclk_marked_level(tmp_path):
    p = tmp_path / "pp_dpm_sclk"
    # the firmware's sampled clock on its own 'S:' line, marked as current
    p.write_text("S: 1834Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) == 1834.0
    # a listed level marked as current
    p.write_text("0: 500Mhz\n1: 2400Mhz *\n")
    assert bench.read_sclk_mhz(str(p)) == 2400.0
    # nothing marked
    p.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(p)) is None


def test_gemm_peak_per_operand_format():
    """Each GEMM row is priced against the peak of the MFMA it issues: E2M1 x E2M1 and the E3M2
    pairs at the MXFP4 rate (FP6 issues at the FP4 rate on gfx950), any E4M3 operand at FP8."""
    MXFP4, MXFP8, FP6P = 0, 1, 2
    assert bench.gemm_peak_tflops(MXFP4, MXFP4) == 10100.0
    assert bench.gemm_peak_tflops(FP6P, FP6P) == 10100.0
    assert bench.gemm_peak_tflops(MXFP8, MXFP4) == 5000.0
    assert bench.gemm_peak_tflops(MXFP8, MXFP8) == 5000.0
    # the E3M2 row of the group-size sweep: 2601 TFLOP/s is 0.26 of the FP4 peak, not 0.52
    assert abs(2601.0 / bench.gemm_peak_tflops(FP6P, FP6P) - 0.2575) < 1e-3
