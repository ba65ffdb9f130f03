"""Low-precision read copies of the checkpoint -- TEST INFRASTRUCTURE ONLY (see
``oracle/__init__.py``).

The "ReplaySSM" README (benefit "Separate state precisions") has non-flush steps read
a low-precision copy of the checkpoint while flushes read and write the
high-precision checkpoint, so that rounding of the copy never enters the recurrence.
The pages name no formats; the ones written here are the library's:

* bf16 and fp16 copies: each fp32 checkpoint element rounded to the nearest value of
  the format, ties to even (a library cast: torch's ``bfloat16`` cast and NumPy's
  ``float16`` cast);
* an fp8 copy in the OCP 8-bit floating point format E4M3 (1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  ``m/8 * 2**-6``; the code with all exponent and mantissa bits set is not a number,
  so the largest finite value is 448 and there are no infinities), with one fp32
  scale per checkpoint row::

      amax  = max_n |h[p, n]|                       (fp32)
      inv   = 448 / amax        (fp32 division; 0 for a zero row)
      code  = nearest E4M3 value of fp32(h * inv), ties to the even code
      scale = amax / 448        (fp32 division; 0 for a zero row)
      value read = code_value * scale

  The sign bit of a code is the sign bit of ``h * inv``.  Inputs never exceed 448 in
  magnitude after scaling except by the last bit of the fp32 product, and such values
  take the largest finite code.

``e4m3_value`` is the format's definition; ``e4m3_encode`` searches the 127
non-negative finite values for the nearest one (ties to the even code), which is the
definition of rounding to nearest even written out.
"""

import numpy as np
import torch


def e4m3_value(code):
    """Value of an E4M3 code (0..255); NaN for the two not-a-number codes."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_POS = np.array([e4m3_value(c) for c in range(0x7F)])     # codes 0x00..0x7e, increasing


def e4m3_encode(x):
    """Codes (uint8) of fp32 values ``x`` rounded to the nearest E4M3 value, ties to
    the even code, magnitudes above 448 to 448."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64)).ravel()
    out = np.empty(a.shape, dtype=np.uint8)
    for i, v in enumerate(a):
        if v >= _POS[-1]:
            c = 0x7E
        else:
            hi = int(np.searchsorted(_POS, v, side="left"))   # _POS[hi-1] < v <= _POS[hi]
            if _POS[hi] == v:
                c = hi
            else:
                lo = hi - 1
                dl, dh = v - _POS[lo], _POS[hi] - v
                c = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        out[i] = c
    sign = np.signbit(x).ravel().astype(np.uint8) << 7
    return (out | sign).reshape(x.shape)


def e4m3_decode(codes):
    return np.vectorize(e4m3_value, otypes=[np.float64])(np.asarray(codes, dtype=np.uint8))


def fp8_copy(h):
    """Row-scaled E4M3 copy of an fp32 checkpoint ``h [..., P, N]``.  Returns
    ``(codes uint8 [..., P, N], scale float32 [..., P])``."""
    h = np.asarray(h, dtype=np.float32)
    amax = np.max(np.abs(h), axis=-1)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(448.0) / amax, np.float32(0.0)).astype(np.float32)
    scaled = (h * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(scaled)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    return codes, scale


def fp8_values(codes, scale):
    """Values read from an fp8 copy (float64)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def bf16_copy(h):
    """bf16 copy as float64 values (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(h, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f16_copy(h):
    """fp16 copy as float64 values (round to nearest even)."""
    return np.asarray(h, dtype=np.float32).astype(np.float16).astype(np.float64)


def copy_error_bound(h, kind, scale=None):
    """Largest |value read - h| elementwise allowed by rounding to nearest: half a unit
    in the last place of the format at |h| (bf16 8 significant bits, fp16 11, E4M3 4 in
    the scaled domain), with the formats' subnormal steps."""
    a = np.abs(np.asarray(h, dtype=np.float64))
    if kind == "bf16":
        return np.ldexp(1.0, -8) * a
    if kind == "f16":
        return np.maximum(np.ldexp(1.0, -11) * a, np.ldexp(1.0, -25))
    if kind == "fp8":
        s = np.asarray(scale, dtype=np.float64)[..., None]
        return np.maximum(np.ldexp(1.0, -4) * a, np.ldexp(1.0, -10) * s)
    raise ValueError(kind)
