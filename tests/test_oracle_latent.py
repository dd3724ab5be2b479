"""Pins of oracle.latent (RMSNorm, RoPE, the finished entry and the indexer key from the main KV)."""

import math

import numpy as np

import oracle
from oracle import latent as lt
from sparse_attention_fp4_kv_amd import workloads as wl


def test_rms_norm_constant_vector_and_scale_invariance():
    x = np.full((1, 512), -3.0)
    g = np.linspace(0.5, 1.5, 512)
    # mean square 9: -3 / sqrt(9 + eps) * g
    y = lt.rms_norm(x, g, 0.0)
    assert np.allclose(y, -g, rtol=0, atol=1e-15)
    y = lt.rms_norm(x, g, 7.0)
    assert np.allclose(y, -3.0 / 4.0 * g, rtol=0, atol=1e-15)
    r = np.random.default_rng(1).standard_normal((4, 512))
    a, b = lt.rms_norm(r, np.ones(512), 0.0), lt.rms_norm(r * 1e3, np.ones(512), 0.0)
    assert np.allclose(a, b, rtol=1e-12, atol=0)
    assert np.allclose(np.sqrt(np.mean(a * a, axis=1)), 1.0, rtol=1e-12)


def test_rope_frequencies_hand_values():
    f = lt.rope_frequencies(10000.0)
    assert f.dtype == np.float32 and f[0] == 1.0
    assert f[16] == np.float32(0.01)  # 10000^(-1/2)
    assert f[31] == np.float32(10000.0 ** (-62 / 64))


def test_rope_identity_at_zero_and_pair_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 512))
    assert np.array_equal(lt.rope(x, [0, 0, 0], 10000.0), x)
    assert np.array_equal(lt.rope(x, [5, 6, 7], 0.0), x)
    y = lt.rope(x, [1, 1000, 1 << 20], 10000.0)
    assert np.array_equal(y[:, :448], x[:, :448])  # only the last 64 channels move
    n0 = x[:, 448::2] ** 2 + x[:, 449::2] ** 2
    n1 = y[:, 448::2] ** 2 + y[:, 449::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


def test_rope_hand_rotation():
    """Pair 0 has frequency 1: at p = 1 it turns by one radian; pair 16 by 0.01 rad at p = 1."""
    x = np.zeros((1, 512))
    x[0, 448], x[0, 449] = 1.0, 0.0
    x[0, 480], x[0, 481] = 0.0, 2.0
    y = lt.rope(x, [1], 10000.0)
    assert abs(y[0, 448] - math.cos(1.0)) < 1e-15 and abs(y[0, 449] - math.sin(1.0)) < 1e-15
    t = float(np.float32(0.01))
    assert abs(y[0, 480] - (-2.0 * math.sin(t))) < 1e-15 and abs(y[0, 481] - 2.0 * math.cos(t)) < 1e-15


def test_rope_dot_depends_on_position_difference():
    """<R(p) a, R(q) b> over the rotated channels is a function of p - q (exact angles: small p, theta with
    power-of-two frequencies so every fp32 angle product is exact)."""
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal((1, 512)), rng.standard_normal((1, 512))
    theta = 2.0 ** 32  # frequencies 2^(-i) : exact in fp32, p * f exact
    d = lambda p, q: float((lt.rope(a, [p], theta)[0, 448:] * lt.rope(b, [q], theta)[0, 448:]).sum())
    assert abs(d(10, 3) - d(107, 100)) < 1e-12
    assert abs(d(0, 0) - float((a[0, 448:] * b[0, 448:]).sum())) < 1e-12
    assert abs(d(5, 5) - d(0, 0)) < 1e-12


def test_finish_reduces_to_plain_pack():
    """gamma = 1, eps = 0, no rotation and an input whose mean square is exactly 1: the finished entry
    is the input, so its pack is the plain pack."""
    rng = np.random.default_rng(4)
    signs = rng.choice([-1.0, 1.0], size=(6, 512))
    c = signs * rng.choice([0.5, 1.0], size=(6, 512))
    # make every row's mean square exactly 1: balance the 0.5 entries with sqrt(7)/2-free values
    c[:, :256] = signs[:, :256] * 0.5
    c[:, 256:] = signs[:, 256:] * math.sqrt(1.75)  # mean of 0.25 and 1.75 = 1
    x, codes, scales, *_ = lt.kv_entry(c, np.arange(6), np.ones(512), 0.0, 0.0)
    assert np.allclose(x, c, rtol=1e-15, atol=0)
    oc, os_ = oracle.fp4.fp4_pack(c.astype(np.float32))
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)


def test_indexer_key_permutation_weights():
    """W_idx = rows of the identity: the key is the selected channels of the dequantized entry, exactly."""
    rng = np.random.default_rng(5)
    st = wl.Streams(5)
    c = wl.latent_rows(st, 0, 0, 7)
    sel = rng.permutation(512)[:128]
    w = np.zeros((128, 512), dtype=np.float32)
    w[np.arange(128), sel] = 1.0
    w_bits = wl.to_bf16_bits(w)
    x, codes, scales, k, kc, ks = lt.kv_entry(c, np.arange(7) + 100, np.full(512, 0.75), 1e-6, 10000.0, w_bits)
    x_hat = oracle.fp4.fp4_unpack(codes, scales)
    assert np.array_equal(k, x_hat[:, sel])
    # the key's own pack is the plain pack of those values (a zero from the sum is +0: -0 entries fold)
    pc, ps = oracle.fp4.fp4_pack((x_hat[:, sel] + 0.0).astype(np.float32))
    assert np.array_equal(kc, pc) and np.array_equal(ks, ps)
    # the stored entry is within one scale step of the finished latent (largest E2M1 half-gap is 1)
    s = np.repeat(oracle.fp4.e4m3_decode(scales), 16, axis=1)
    assert np.all(np.abs(x_hat - x) <= s)


def test_finished_entry_range_bound():
    """The pages' range argument: with |gamma| <= 1 the finished latent has L2 norm <= sqrt(512), so no
    channel exceeds sqrt(512) ~ 22.6, far inside the 2688 the format represents."""
    st = wl.Streams(6)
    c = wl.latent_rows(st, 0, 0, 64)  # outlier channels x20
    g = np.random.default_rng(6).uniform(-1, 1, 512)
    x = lt.finish_latent(c, np.arange(64) * 977, g, 1e-6, 10000.0)
    assert np.all(np.linalg.norm(x, axis=1) <= math.sqrt(512) * (1 + 1e-12))
    assert np.max(np.abs(x)) <= 22.63


def test_rope_angle_rounded_to_fp32():
    """The angle is the fp32 product fl32(p * fl32(f)), not the exact product.  Worked by hand for pair
    16 (f = 10000^(-1/2) = 0.01) at p = 7: fl32(0.01) = 5368709 * 2^-29 (an odd 23-bit integer); 7 times
    that is 37580963 * 2^-29, a 26-bit integer that fp32 cannot hold; its 24-bit rounding is
    37580963 / 4 = 9395240.75 -> 9395241 (nearest), so the angle is 9395241 * 2^-27 =
    0.070000000298023223876953125, while the exact product is 0.06999999843537807..."""
    f = lt.rope_frequencies(10000.0)
    assert int(f[16].view(np.uint32)) == 0x3C23D70A  # 5368709 * 2^-29
    t = lt.rope_angles([7], 10000.0)[0, 16]
    assert float(t) == 9395241 * 2.0 ** -27 == 0.070000000298023223876953125
    exact = 37580963 * 2.0 ** -29
    assert float(t) != exact  # a float64 product would fail this
    x = np.zeros((1, 512))
    x[0, 480], x[0, 481] = 1.0, 0.0
    y = lt.rope(x, [7], 10000.0)
    assert abs(y[0, 480] - math.cos(9395241 * 2.0 ** -27)) < 1e-16
    assert abs(y[0, 481] - math.sin(9395241 * 2.0 ** -27)) < 1e-16
    assert abs(y[0, 481] - math.sin(exact)) > 1e-10  # the two readings are told apart
    # a large position: p = 2^20 + 3 on pair 1 (f = fl32(10000^(-1/32)))
    f1 = int(f[1].view(np.uint32))
    mant, ex = (f1 & 0x7FFFFF) | 0x800000, ((f1 >> 23) & 0xFF) - 150  # f = mant * 2^ex
    prod = ((1 << 20) + 3) * mant  # exact integer product, 44 bits
    sh = prod.bit_length() - 24
    q, r = divmod(prod, 1 << sh)
    q += 1 if (2 * r > (1 << sh) or (2 * r == (1 << sh) and q & 1)) else 0  # round to nearest even
    assert float(lt.rope_angles([(1 << 20) + 3], 10000.0)[0, 1]) == q * 2.0 ** (ex + sh)
