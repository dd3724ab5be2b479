"""Pins of oracle.swa (FP8 window entries, the window, and the merge with the global branch)."""

import numpy as np

import oracle
from oracle import swa
from sparse_attention_fp4_kv_amd import workloads as wl


def test_fp8_pack_round_trips_every_code():
    """Rows built from every finite E4M3 value times a power-of-two scale (amax 448 exactly) pack back to
    the same bytes and decode to the same values."""
    vals = oracle.fp4.e4m3_decode(np.arange(0, 0x7F))  # 0 .. 448
    row = np.concatenate([vals, -vals[1:]])             # 253 values, amax 448
    row = np.pad(row, (0, 256 - row.size))
    for k in (-3, 0, 5):
        x = (row * 2.0 ** k).astype(np.float32)[None]
        codes, s = swa.swa_pack(x)
        assert s[0] == np.float32(2.0 ** k)
        assert np.array_equal(swa.swa_unpack(codes, s), x.astype(np.float64))
        assert np.array_equal(codes[0, :127], np.arange(0, 0x7F, dtype=np.uint8))
        assert np.array_equal(codes[0, 127:253], (np.arange(1, 0x7F) | 0x80).astype(np.uint8))


def test_fp8_pack_error_bound_and_zero_row():
    st = wl.Streams(90)
    x = wl.latent_rows(st, 0, 0, 50)
    codes, s = swa.swa_pack(x)
    xh = swa.swa_unpack(codes, s)
    # E4M3: 3 mantissa bits -> within half a step (2^-4 relative) above the subnormal range, 2^-10 s below it
    err = np.abs(xh - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6))
    assert np.all(np.max(np.abs(xh), axis=1) == 448.0 * s.astype(np.float64))  # amax maps to 448 exactly
    c0, s0 = swa.swa_pack(np.zeros((2, 512), np.float32))
    assert not c0.any() and not s0.any()


def test_window_positions_and_slots():
    assert swa.window_positions(0).size == 0
    assert np.array_equal(swa.window_positions(5), np.arange(5))
    w = swa.window_positions(1000)
    assert w[0] == 872 and w[-1] == 999 and w.size == 128
    assert sorted(swa.window_slot(w).tolist()) == list(range(128))  # a full ring holds every slot once
    # hand values of the ring slot (position mod 128): a new token overwrites the entry 128 positions back
    assert swa.window_slot([0, 1, 127, 128, 129, 999, 1000]).tolist() == [0, 1, 127, 0, 1, 103, 104]
    assert swa.window_slot(1000) == swa.window_slot(1000 - 128)
    # the window slides by one position per token: the oldest position leaves as the new one enters
    assert np.array_equal(swa.window_positions(1001)[:-1], swa.window_positions(1000)[1:])
    assert swa.window_positions(128).tolist() == list(range(128)) and swa.window_positions(129)[0] == 1


def test_merge_equals_attention_over_the_union():
    rng = np.random.default_rng(91)
    st = wl.Streams(91)
    q = wl.q_heads(st, 0, 1, 16, 576)[0]
    cg = rng.standard_normal((40, 512))
    rg = rng.standard_normal((40, 64))
    cs = rng.standard_normal((25, 512))
    sigma = 1 / np.sqrt(576)
    og, lg = oracle.attention.sparse_attention(q, cg, sigma, rope_sel=rg)
    os_, ls = swa.swa_attention(q, cs, sigma)
    om, lm = swa.merge(og, lg, os_, ls)
    # directly: one softmax over both sets (window entries have no rope part)
    ou, lu = oracle.attention.sparse_attention(q, np.concatenate([cg, cs]), sigma,
                                               rope_sel=np.concatenate([rg, np.zeros((25, 64))]))
    assert np.allclose(om, ou, rtol=1e-12, atol=1e-12) and np.allclose(lm, lu, rtol=1e-12, atol=1e-12)
    # an empty branch leaves the other unchanged; both empty -> 0, -inf
    e_o, e_l = np.zeros((16, 512)), np.full(16, -np.inf)
    o1, l1 = swa.merge(og, lg, e_o, e_l)
    assert np.array_equal(o1, og) and np.array_equal(l1, lg)
    o2, l2 = swa.merge(e_o, e_l, os_, ls)
    assert np.allclose(o2, os_, rtol=1e-15) and np.array_equal(l2, ls)
    o3, l3 = swa.merge(e_o, e_l, e_o, e_l)
    assert not o3.any() and np.all(np.isneginf(l3))
