"""Host checks of arithmetic identities the quantizer kernel relies on.

The activation scale is s = bf16(fl32(A / 7)) with A = max |x_hat| a bf16 value
(mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
4-Bit-Quantisierung", section "Nunchaku und SVDQuant": symmetric 4-bit groups).
The kernel forms it as bf16(fl32(A * fl32(1/7))), one multiply instead of an
IEEE division.  The two fp32 values differ in the last bit for about half of
all A, so the identity only holds after the bf16 rounding; it is checked here
for every non-negative finite bf16 A.
"""
import numpy as np

import oracle as O


def _bf16_values(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_scale_by_multiply_equals_scale_by_division_for_every_bf16():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 ... largest finite
    A = _bf16_values(bits)
    by_div = O.f32_to_bf16(A / np.float32(7.0))
    by_mul = O.f32_to_bf16(A * np.float32(1.0 / 7.0))
    assert by_div.dtype == by_mul.dtype == np.uint16
    assert np.array_equal(by_div, by_mul)
    # the fp32 intermediates do differ: the identity is not trivial
    assert np.count_nonzero((A / np.float32(7.0)) != (A * np.float32(1.0 / 7.0))) > 1000


def test_reciprocal_range_guard_covers_all_scales_of_ordinary_data():
    """The kernel's fast reciprocal is used for s in [2^-100, 2^100]; every
    bf16 A in [7 * 2^-100, 2^100] gives such an s."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    A = _bf16_values(bits).astype(np.float64)
    s = O.bf16_to_f64(O.f32_to_bf16((A / 7.0).astype(np.float32)))
    sel = (A >= 7 * 2.0 ** -100) & (A <= 2.0 ** 100)
    assert np.all((s[sel] >= 2.0 ** -100) & (s[sel] <= 2.0 ** 100))
