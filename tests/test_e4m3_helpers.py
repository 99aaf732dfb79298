"""The FP8 E4M3 facts the parity tests rely on, pinned to the format's
definition (OCP 8-bit floating point, E4M3: exponent bias 7, 3 fraction bits,
no infinities, only S.1111.111 is NaN, largest finite value 448) rather than
to torch: torch's decode of every code, the e4m3 spacing the tolerance uses,
and torch's rounding of fp32 to e4m3, which makes the test inputs."""
import numpy as np
import torch

from gpu_checks import e4m3_expected, e4m3_ulp


def definition_value(code):
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_torch_decodes_every_code_as_defined():
    got = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    want = np.array([definition_value(c) for c in range(256)])
    both_nan = np.isnan(got) & np.isnan(want)
    assert (both_nan | (got == want)).all()
    assert np.nanmax(want) == 448.0 and np.isnan(want).sum() == 2


def test_ulp_is_the_gap_to_the_next_value():
    vals = np.array(sorted(definition_value(c) for c in range(127)))  # 0 ... 448
    gaps = vals[1:] - vals[:-1]
    np.testing.assert_array_equal(e4m3_ulp(vals[:-1]), gaps)
    np.testing.assert_array_equal(e4m3_ulp(-vals[:-1]), gaps)
    assert e4m3_ulp(np.array([0.0]))[0] == 2.0 ** -9


def test_saturated_expectation():
    r = np.array([500.0, -1e9, 447.0, np.nan, -448.0])
    e = e4m3_expected(r)
    assert e[0] == 448.0 and e[1] == -448.0 and e[2] == 447.0 and np.isnan(e[3]) and e[4] == -448.0


def test_torch_rounds_to_nearest_even():
    """Inputs are drawn in fp32 and rounded to e4m3 by torch: nearest value,
    ties to the even code, as the definition and round-to-nearest-even fix."""
    vals = np.array([definition_value(c) for c in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2  # exact in fp32
    got = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)  # the even neighbour
    np.testing.assert_array_equal(got, want)
    # just off a midpoint: the nearer value
    up = np.nextafter(mids.astype(np.float32), np.float32(1e9))
    got = torch.from_numpy(up).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, lo + 1)
