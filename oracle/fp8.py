"""FP8 (E4M3) key/value cache codes for the decode path (test infrastructure
only, like the rest of this package).

The pages size the KV cache with an FP8 column beside BF16 and leave scale
factors out of the count (Muse Spark Open deep dive, section 7.2, the KV
cache table and its note).  The cache convention here fills in what they
leave open:

* a cached value x of one (page, KV head) -- or of one (sequence, KV head)
  for the ring -- is stored as the E4M3 code of x / scale, with the division
  done in IEEE fp32 and scale an fp32 number the caller supplies per
  (page, KV head);
* E4M3 is the OCP 8-bit format: 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals, no infinities, codes 0x7F / 0xFF are NaN, the
  largest finite magnitude is 448;
* encoding rounds to the nearest representable value, ties to the code with
  an even mantissa, and saturates finite values beyond 448 to +-448 (the
  cache never stores NaN for a finite input);
* decoding is exact: value(code) * scale.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6          # subnormal
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALUES = e4m3_values()
_POS = _VALUES[:127]          # codes 0x00 .. 0x7E: 0 .. 448, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Codes of x: nearest finite E4M3 value, ties to even mantissa,
    saturating at +-448; NaN -> 0x7F.  The sign is kept (-0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for n, v in enumerate(flat):
        if np.isnan(v):
            out[n] = 0x7F
            continue
        a = min(abs(v), E4M3_MAX)
        i = int(np.searchsorted(_POS, a))          # _POS[i-1] < a <= _POS[i]
        if i == 0:
            code = 0
        elif i >= 127:
            code = 126
        else:
            lo, hi = _POS[i - 1], _POS[i]
            if a - lo < hi - a:
                code = i - 1
            elif a - lo > hi - a:
                code = i
            else:                                   # tie: even mantissa
                code = i - 1 if (i - 1) % 2 == 0 else i
        if np.signbit(v):
            code |= 0x80
        out[n] = code
    return out.reshape(x.shape)


def quantize(x, scale) -> np.ndarray:
    """Cache codes of values x with the given scale (division in fp32)."""
    q = np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32)
    return e4m3_encode(q.astype(np.float32))


def dequantize(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)
