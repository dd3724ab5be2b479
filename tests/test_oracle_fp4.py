"""Pins of the oracle's FP4 format code against facts outside the oracle.

- E2M1 table and E4M3 facts from tests/golden/fp4_format.json (format
  definitions named by the pages, and the pages' 448 x 6 = 2688 range).
- E4M3 decode of all 256 codes against torch.float8_e4m3fn (a library routine).
- E4M3 encode against torch's float32 -> float8_e4m3fn rounding (round to
  nearest even) for every value below the saturation boundary tested.
- An exhaustive boundary sweep of the E2M1 element decision against an exact
  rational nearest-point search written here with fractions.Fraction.
- Hand-worked pack groups (tests/golden/pack_groups.json).
- The quantization error bound and the bytes-per-row arithmetic.
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from oracle import fp4


def _f(x):
    return float.fromhex(x) if isinstance(x, str) and x.startswith("0x") else x


def test_e2m1_table(golden):
    g = golden("fp4_format.json")
    assert list(fp4.e2m1_decode(np.arange(8))) == g["e2m1_magnitudes"]["value"]
    assert list(fp4.e2m1_decode(np.arange(8, 16))) == [-v for v in g["e2m1_magnitudes"]["value"]]
    assert fp4.E2M1_MAX == g["e2m1_max"]["value"]
    assert fp4.E4M3_MAX * fp4.E2M1_MAX == g["format_range"]["value"]
    assert fp4.GROUP == g["channels_per_scale"]["value"]


def test_e4m3_known_codes(golden):
    g = golden("fp4_format.json")
    for code, val in g["e4m3_known_codes"]["value"].items():
        assert fp4.e4m3_decode(int(code, 16)) == val, code
    assert fp4.e4m3_decode(0x7E) == g["e4m3_max"]["value"]
    assert np.isnan(fp4.e4m3_decode(0x7F)) and np.isnan(fp4.e4m3_decode(0xFF))


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp4.e4m3_decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))
    assert np.sum(both_nan) == 2


def test_e4m3_round_trip_all_finite_codes():
    vals = fp4.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)
    assert np.array_equal(fp4.e4m3_encode(vals), np.arange(0x7F, dtype=np.uint8))


def test_e4m3_rounding_cases(golden):
    for v, code in golden("fp4_format.json")["e4m3_rounding_cases"]["value"]:
        assert int(fp4.e4m3_encode(np.float64(v))) == int(code, 16), v


def _e4m3_exact_nearest(v):
    """Nearest finite E4M3 code by exact rational search; ties to the even code; saturate."""
    fv = Fraction(v)
    best = None
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        val = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        d = abs(fv - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e4m3_encode_exact_search_at_midpoints():
    vals = fp4.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    probe = []
    for m in mids:
        m32 = np.float32(m)
        assert float(m32) == m  # midpoints are exact in fp32
        probe += [np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(1e9))]
    rng = np.random.default_rng(5)
    probe += list(np.float32(np.exp(rng.uniform(math.log(1e-4), math.log(600.0), size=400))))
    probe = np.array(probe, dtype=np.float32)
    ours = fp4.e4m3_encode(probe.astype(np.float64))
    for v, c in zip(probe, ours):
        assert int(c) == _e4m3_exact_nearest(float(v)), float(v)


def test_e4m3_encode_matches_torch_below_saturation():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        np.float32(np.exp(rng.uniform(math.log(1e-6), math.log(463.0), size=20000))),
        np.float32(fp4.e4m3_decode(np.arange(0x7F))),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = fp4.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ref, ours)


def _e2m1_exact_nearest(ax, s):
    q = Fraction(ax) / Fraction(s)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    best = None
    for c, g in enumerate(grid):
        d = abs(q - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_boundary_sweep_exhaustive():
    """All 126 non-zero scales x 7 decision thresholds x {prev, equal, next} fp32 x sign."""
    scales = fp4.e4m3_decode(np.arange(1, 0x7F))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    ax_list, s_list = [], []
    for s in scales:
        for m in mids:
            t = np.float32(m * s)
            assert float(t) == m * s
            for v in (np.nextafter(t, np.float32(0)), t, np.nextafter(t, np.float32(1e9))):
                ax_list.append(float(v))
                s_list.append(float(s))
        for v in (6.0 * s, 7.0 * s, 0.0):  # saturation region and zero
            ax_list.append(float(np.float32(v)))
            s_list.append(float(s))
    ax = np.array(ax_list)
    sv = np.array(s_list)
    ours = fp4.e2m1_quantize_magnitude(ax, sv)
    for a, s, c in zip(ax_list, s_list, ours):
        assert int(c) == _e2m1_exact_nearest(a, s), (a, s)


def _parse(v):
    if v == "-0":
        return -0.0
    return float(v)


def test_pack_hand_worked_groups(golden):
    for g in golden("pack_groups.json")["groups"]:
        x = np.array([[_parse(v) for v in g["x"]]], dtype=np.float32)
        codes, scales = fp4.fp4_pack(x)
        assert int(scales[0, 0]) == int(g["scale"], 16), g["name"]
        assert [int(c) for c in codes[0]] == [int(c, 16) for c in g["codes"]], g["name"]


def test_pack_error_bound_and_layout():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, [3, 77, 200, 301, 450]] *= 20
    codes, scales = fp4.fp4_pack(x)
    assert codes.shape == (64, 256) and scales.shape == (64, 32)
    assert fp4.packed_row_bytes(512) == 288
    deq = fp4.fp4_unpack(codes, scales)
    s = np.repeat(fp4.e4m3_decode(scales), 16, axis=-1)
    q = np.abs(x.astype(np.float64)) / s
    # grid step around the quotient: 0.5 below 2, 1 below 4, 2 above
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    inside = q <= 6
    err = np.abs(x.astype(np.float64) - deq)
    assert np.all(err[inside] <= 0.5 * step[inside] * s[inside])
    # values above 6 s (only possible when the scale rounded down) saturate at 6 s
    assert np.all(np.abs(deq[~inside]) == 6 * s[~inside])
    # low nibble is the even channel
    nib0 = codes[:, 0] & 0xF
    assert np.array_equal(fp4.e2m1_decode(nib0) * s[:, 0], deq[:, 0])


def test_pack_scale_definition_per_group():
    """Scale byte == E4M3(fl32(amax/6)) checked against torch's fp8 rounding."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((256, 64)) * np.exp(rng.uniform(-6, 6, size=(256, 1)))).astype(np.float32)
    _, scales = fp4.fp4_pack(x)
    amax = np.abs(x.reshape(256, 4, 16)).max(axis=-1)
    v = (amax / np.float32(6)).astype(np.float32)
    v = np.minimum(v, np.float32(448))  # torch's conversion is not saturating; clamp first
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, scales)


def test_bound_sqrt512_fits_range(golden):
    g = golden("fp4_format.json")
    assert abs(math.sqrt(g["latent_channels"]["value"]) - g["per_channel_bound"]["value"]) < 1e-12
    # a group at the per-channel bound packs without saturating the scale
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = np.float32(g["per_channel_bound"]["value"])
    codes, scales = fp4.fp4_pack(x)
    assert fp4.e4m3_decode(scales[0, 0]) < fp4.E4M3_MAX
    assert (codes[0, 0] & 0xF) == 7  # the maximum lands on the top grid point
