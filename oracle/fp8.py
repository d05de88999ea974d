"""OCP FP8 E4M3FN decoding -- oracle (test infrastructure only).

The FP8 attention the pages describe ("How FLUX 3 Image Klein was made 3-4x
faster on NVIDIA Blackwell", section "Method 2", table of attention methods)
does not name the format; this library reads it as the OCP 8-bit floating-point
E4M3 format without infinities (E4M3FN): 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the pattern
S.1111.111 is NaN; the largest finite magnitude is 448.

Parity: pinned by tests on all 256 codes against torch.float8_e4m3fn and against
hand-checked spec values (tests/golden/e4m3_spec_values.json).
"""

import numpy as np


def _decode_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _decode_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 values of uint8 E4M3FN codes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
