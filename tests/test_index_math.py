"""The kernels' workgroup coordinates come from a division through the hardware
reciprocal with one integer correction (``udiv23`` in ``ssd_device.hpp``):
q = trunc(float(n) * rcp(float(d))), r = n - q d, q += (r >= d) - (r < 0).
This checks the error argument behind it on the host, for every n below 2^23:
with the reciprocal off by up to one ulp either way (the hardware's stated
accuracy), the corrected quotient equals floor(n / d).  The divisors include
the small ones (head counts, p tiles, groups), powers of two and the largest
ones the bound allows."""
import numpy as np


def _udiv23_model(n, d, rcp):
    p = (n.astype(np.float32) * np.float32(rcp)).astype(np.float32)
    q = p.astype(np.int64)
    r = n - q * d
    return q + (r >= d) - (r < 0)


def test_reciprocal_division_is_exact_below_2_23():
    n = np.arange(0, 1 << 23, dtype=np.int64)
    for d in [1, 2, 3, 5, 6, 7, 24, 32, 63, 80, 97, 127, 1000, 4097, 65535, (1 << 22) + 1, (1 << 23) - 1]:
        r0 = np.float32(1.0) / np.float32(d)
        rcps = [r0] if d in (1, 2) else [r0, np.nextafter(r0, np.float32(0)), np.nextafter(r0, np.float32(1))]
        for rcp in rcps:   # powers of two have an exact reciprocal
            q = _udiv23_model(n, d, rcp)
            bad = np.flatnonzero(q != n // d)
            assert bad.size == 0, (d, rcp, n[bad[:5]])
