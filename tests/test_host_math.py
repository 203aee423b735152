"""Host-side checks of arithmetic claims the kernels rely on."""
import numpy as np


def test_reciprocal_small_division_is_exact():
    # The 16-bit implicit data-gradient loader decodes a stage's tap as
    # int((n + 0.5) * rcp(d)) with the hardware reciprocal (within 1 ulp);
    # the host only enables it for n < 2^20 and d <= 1024.  The quotient can
    # only go wrong next to a multiple of d, so those n are checked, with
    # the reciprocal rounded down, exactly and up.
    f = np.float32
    for d in range(1, 1025):
        q = np.arange(0, (1 << 20) // d + 2, dtype=np.int64)
        n = np.concatenate([q * d - 1, q * d, q * d + d - 1])
        n = n[(n >= 0) & (n < (1 << 20))]
        r0 = f(1.0) / f(d)
        for r in (np.nextafter(r0, f(0)), r0, np.nextafter(r0, f(2))):
            got = np.floor((n.astype(np.float32) + f(0.5)) * r).astype(np.int64)
            assert np.array_equal(got, n // d), d
