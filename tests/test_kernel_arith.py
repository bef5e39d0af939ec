"""Host checks of arithmetic identities the kernels rely on (no GPU).

The Gumbel noise draws u = ((w >> 9) + 0.5) 2^-23 from a 32-bit generator word
w (Gumbel-max sampling with an explicit key).  The kernels build u without an
integer conversion: the 23 word bits go under the exponent of 1.0, giving the
float 1 + m 2^-23 (m = w >> 9), and 1 - 2^-24 is subtracted.  The difference
(2m + 1) 2^-24 has a 24-bit significand, so float32 subtraction returns it
exactly: checked here for every m.
"""
import numpy as np


def test_uniform_from_word_bit_construction_is_exact():
    m = np.arange(1 << 23, dtype=np.uint32)
    one_plus = (m | np.uint32(0x3F800000)).view(np.float32)
    u = one_plus - np.float32(1.0 - 2.0 ** -24)
    assert u.dtype == np.float32
    want = (m.astype(np.float64) + 0.5) * 2.0 ** -23
    assert np.array_equal(u.astype(np.float64), want)
    assert u.min() > 0 and u.max() < 1
