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
