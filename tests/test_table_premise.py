"""The facts about the sigmoid that the kernels' lookup tables rest on,
checked on the oracle's correctly rounded sigmoid for every bf16 gate (CPU).

The kernels tabulate sigma for the bf16 magnitudes 2^-25 .. 127.5 and clamp
any other magnitude into that range; the 16 KiB form of the table keeps
sigma(-|g|) and recovers sigma(+|g|) as RN(1 - sigma(-|g|)) plus a correction
of -1, 0 or +1 ulp stored in the two top bits of sigma(-|g|)."""
import numpy as np

import oracle

FIRST, LAST = 0x3300, 0x42FF  # bf16 bits of 2^-25 and 127.5


def _g(m):
    return float(np.uint32(m << 16).view(np.float32))


def _bits(v):
    return int(np.float32(v).view(np.uint32))


def test_correction_fits_in_two_bits_for_every_tabulated_magnitude():
    seen = set()
    for m in range(FIRST, LAST + 1):
        g = _g(m)
        sn = np.float32(oracle.sigmoid(-g))
        sp = np.float32(oracle.sigmoid(g))
        assert _bits(sn) >> 30 == 0, (hex(m), float(sn))          # sigma(-|g|) <= 0.5: two free top bits
        corr = _bits(sp) - _bits(np.float32(np.float32(1.0) - sn))  # RN(1 - s) in fp32
        assert corr in (-1, 0, 1), (hex(m), corr)
        seen.add(corr)
    assert seen == {-1, 0, 1}


def test_clamping_the_magnitude_into_the_table_is_exact():
    lo_p, lo_n = oracle.sigmoid(_g(FIRST)), oracle.sigmoid(-_g(FIRST))
    hi_p, hi_n = oracle.sigmoid(_g(LAST)), oracle.sigmoid(-_g(LAST))
    assert lo_p == lo_n == 0.5 and hi_p == 1.0 and hi_n == 0.0
    for m in list(range(0, FIRST)) + list(range(LAST + 1, 0x7F80)):
        g = _g(m)
        want_p, want_n = (lo_p, lo_n) if m < FIRST else (hi_p, hi_n)
        assert oracle.sigmoid(g) == want_p and oracle.sigmoid(-g) == want_n, hex(m)
