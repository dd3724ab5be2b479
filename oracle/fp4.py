"""FP4 KV format of the oracle: E2M1 elements with one E4M3 scale per 16 channels.

Source: [P1] section "FP4 KV cache" -- the main KV cache is stored as FP4 E2M1
values with one E4M3 scale for every 16 channels (NVFP4 without its second,
global scale level); the representable magnitude reaches 448 x 6 = 2688; the
cache is dequantized before attention, so no FP4 matmul is involved.  The same
format is restated in [P3] "규모와 구조" and [P4] section 3.

What the pages leave open, and the reading taken here (each one is listed in
the design notes as a reading of the pages):
  * E4M3 variant: the maximum 448 fixes the OCP "FN" variant (bias 7, no
    infinities, 0x7F/0xFF are NaN, largest finite 0x7E = 448).
  * Scale: s = E4M3_RNE(fl32(amax / 6)), i.e. the quotient is formed in IEEE
    fp32 first, then rounded to the nearest E4M3 value with ties to the even
    code, saturating at 448.  amax == 0, or a quotient that rounds to zero,
    gives s = 0.
  * Elements: the nearest point of the E2M1 grid {0,.5,1,1.5,2,3,4,6} to the
    exact quotient |x| / s, ties to the even code, saturating at 6.  With s = 0
    every nibble of the group is 0.
  * Sign: the sign bit of x is kept when s > 0 (so -0.0 and tiny negatives give
    nibble 0x8).
  * Byte layout: byte j of a row holds channel 2j in its low nibble and
    channel 2j+1 in its high nibble; scales are a separate byte array with one
    byte per 16-channel group g (channels 16g .. 16g+15).
  * Inputs are finite (the generators never produce NaN or Inf).

Parity pins (tests/test_oracle_fp4.py): the E2M1 table; every E4M3 code's
value checked against torch.float8_e4m3fn; encode(decode(c)) == c for all 127
finite non-negative codes; an exhaustive boundary sweep (every non-zero scale x
every decision threshold x {prev, equal, next} fp32 x sign) against an exact
rational nearest-point search; hand-worked groups in tests/golden/.
"""

import numpy as np

GROUP = 16  # channels per E4M3 scale ([P1] "FP4 KV cache")

# E2M1 magnitudes indexed by the low 3 bits of a nibble (s e1 e0 m): exponent
# bias 1, one subnormal (e=0, m=1 -> 0.5).  Largest value 6.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_decode(nibbles):
    """Value of each 4-bit E2M1 code (sign bit 3, magnitude bits 0-2)."""
    n = np.asarray(nibbles, dtype=np.int64) & 0xF
    mag = E2M1_MAGNITUDES[n & 7]
    return np.where((n & 8) != 0, -mag, mag)


def e4m3_decode(codes):
    """Value of each E4M3FN byte (s eeee mmm, bias 7); NaN for 0x7F / 0xFF.

    exponent field 0: m/8 * 2^-6 (subnormal); otherwise (1 + m/8) * 2^(e-7).
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# The 127 finite non-negative E4M3 values, in code order (strictly increasing).
_E4M3_POS = e4m3_decode(np.arange(0, E4M3_MAX_CODE + 1))


def e4m3_encode(v):
    """Nearest non-negative E4M3FN code to each fp32 value v >= 0.

    Round-to-nearest with ties to the even code; values above 448 saturate to
    0x7E (448).  Implemented as a search over the table of all finite codes.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3_encode expects finite non-negative values")
    hi = np.searchsorted(_E4M3_POS, v, side="left")  # first code with value >= v
    hi = np.minimum(hi, E4M3_MAX_CODE)
    lo = np.maximum(hi - 1, 0)
    d_lo = v - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - v
    exact = _E4M3_POS[hi] == v
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    code = np.where(v >= E4M3_MAX, E4M3_MAX_CODE, code)
    return code.astype(np.uint8)


# Midpoints between neighbouring E2M1 magnitudes; midpoint k separates code k
# from code k+1.  On a tie the even one of the two codes is taken.
_E2M1_MIDPOINTS = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0  # .25 .75 1.25 1.75 2.5 3.5 5


def e2m1_quantize_magnitude(ax, s):
    """E2M1 magnitude code (0..7) nearest to the exact quotient ax / s.

    ax: |x| as float64 holding fp32 values; s: positive scale values.
    Every midpoint * s is exact in float64 (at most 7 significant bits), so
    comparing ax against it decides the nearest grid point exactly: the code
    is the number of midpoints below ax, and a value sitting exactly on a
    midpoint goes to the even code of the pair.  Values beyond 6*s saturate to
    code 7 because there is no midpoint above it.
    """
    ax = np.asarray(ax, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    code = np.zeros(np.broadcast(ax, s).shape, dtype=np.int64)
    for k, mid in enumerate(_E2M1_MIDPOINTS):
        t = mid * s
        upper_is_even = (k + 1) % 2 == 0
        code += (ax > t) | ((ax == t) & upper_is_even)
    return code


def fp4_pack(x):
    """Pack rows of fp32 channels into (codes, scales).

    x: float32 array [..., C] with C % 16 == 0.
    returns codes uint8 [..., C/2], scales uint8 [..., C/16] (E4M3FN bytes).
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("fp4_pack expects float32 input (the cache's latent precision)")
    C = x.shape[-1]
    if C % GROUP != 0:
        raise ValueError("channel count must be a multiple of 16")
    lead = x.shape[:-1]
    g = x.reshape(lead + (C // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)                      # exact in fp32
    quotient = (amax / np.float32(6.0)).astype(np.float32)  # IEEE fp32 division
    scode = e4m3_encode(quotient.astype(np.float64))
    s = e4m3_decode(scode)                                 # 0 when the code is 0
    ax = np.abs(g).astype(np.float64)
    mag = e2m1_quantize_magnitude(ax, s[..., None])
    sign = np.signbit(g).astype(np.int64)
    nib = (sign << 3) | mag
    nib = np.where((s == 0)[..., None], 0, nib)
    nib = nib.reshape(lead + (C,))
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return codes, scode.astype(np.uint8)


def fp4_unpack(codes, scales):
    """Dequantize (codes, scales) to float64 values [..., C]; exact in fp32 too."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = codes & 0xF
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals = e2m1_decode(nib)
    s = e4m3_decode(scales)
    C = vals.shape[-1]
    s_per_ch = np.repeat(s, GROUP, axis=-1)
    assert s_per_ch.shape[-1] == C
    return vals * s_per_ch


def packed_row_bytes(channels):
    """Bytes of one packed row: C/2 nibble bytes plus C/16 scale bytes."""
    return channels // 2 + channels // GROUP
