"""Storage codecs written from the format definitions (test infrastructure only).

bf16: the upper 16 bits of an IEEE-754 binary32 value (1 sign, 8 exponent,
7 fraction bits).  Decoding is exact; encoding rounds to nearest, ties to even.

OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
no infinities, S.1111.111 is NaN, largest finite magnitude 1.75 * 2^8 = 448,
subnormals m * 2^-9.  The pages name FP8 as the precision of most matrix
products ([LKVC] "FP8/FP32 Mixed Precision"); the pages do not spell out a
latent-cache quantisation, and the per-token scaled one used here is a
reading of that passage.

Pins: tests compare both codecs with torch's bfloat16 / float8_e4m3fn casts on
CPU over every code and over random values (a library routine as the pin).
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float values to bf16 bit patterns, nearest-even.

    The value is first taken to binary32 (exact for every value stored here,
    which are all binary32 to begin with), then its low 16 bits are
    rounded away with ties going to the even result.  NaN maps to 0x7FC0.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = r.astype(np.uint16)
    r[np.isnan(f)] = np.uint16(0x7FC0)
    return r


def _e4m3_table():
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()
# positive finite codes 0x00..0x7E in increasing value order
_E4M3_POS = _E4M3[:0x7F]


def e4m3_bits_to_f64(bits):
    """Decode OCP e4m3 bit patterns (uint8) to float64 with a 256-entry table."""
    return _E4M3[np.asarray(bits, dtype=np.uint8).astype(np.intp)]


def f64_to_e4m3_bits(x):
    """Encode to OCP e4m3, nearest-even, saturating finite values at +-448.

    NaN maps to 0x7F.  Out-of-range values saturate (rather than becoming
    NaN), a choice the pages leave open; the quantiser's inputs never exceed
    448 in magnitude after scaling.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")      # first value >= mag
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _E4M3_POS[hi] - mag
    d_lo = mag - _E4M3_POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    code[np.isnan(x)] = np.uint8(0x7F)
    return code
