"""GPU parity of the sliding-window branch: FP8 window append (bit-exact), the window attention merged
with the global branch (one softmax over both sets of entries) against the oracle, and the same result from
the attention call that takes the window as extra splits."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import ATTN_TOL, LSE_TOL, build_tables, fill_layer, make_batch, oracle_attention_rows, to_dev

pytestmark = pytest.mark.gpu


def test_swa_append_bit_exact():
    st = wl.Streams(100)
    B = 5
    ring = csa2.SwaRing(B + 2)
    pos = np.array([0, 5, 127, 300, -1], dtype=np.int32)
    x = wl.latent_rows(st, 1, 0, B)
    x[1] = 0.0  # an all-zero row: scale 0, codes 0
    csa2.csa2_swa_append(ring, to_dev(pos), to_dev(x))
    torch.cuda.synchronize()
    codes, scales = ring.codes.cpu().numpy(), ring.scales.cpu().numpy()
    oc, os_ = oracle.swa.swa_pack(x)
    touched = np.zeros((B + 2, 128), dtype=bool)
    for b in range(B):
        if pos[b] < 0:
            continue
        s = int(oracle.swa.window_slot(pos[b]))
        touched[b, s] = True
        assert np.array_equal(codes[b, s], oc[b]) and scales[b, s] == os_[b], b
    assert not codes[~touched].any() and not scales[~touched].any()


def _fill_window(ring, lat_win, seq_lens, skip_last=False):
    """Append every window position of every sequence through the GPU append (one call per position index);
    skip_last leaves out each sequence's last position (n - 1)."""
    B = len(seq_lens)
    W = max(min(n, 128) for n in seq_lens)
    for j in range(W):
        pos = np.array([n - min(n, 128) + j if j < min(n, 128) - (1 if skip_last else 0) else -1 for n in seq_lens],
                       dtype=np.int32)
        rows = np.stack([lat_win[b][j] if pos[b] >= 0 else np.zeros(512, np.float32) for b in range(B)])
        csa2.csa2_swa_append(ring, to_dev(pos), to_dev(rows))


@pytest.mark.parametrize("rope_dim,heads", [(0, 64), (64, 64), (0, 16), (64, 128)])
def test_swa_merge_matches_union_attention(rope_dim, heads):
    st = wl.Streams(101 + rope_dim + heads)
    seq_lens = [1000, 50, 128, 3000, 1]
    B, K = len(seq_lens), 256
    tables, nb = build_tables(st, seq_lens, True)
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)]
    ropes = [wl.rope_rows(st, 0, b, n, rope_dim) for b, n in enumerate(seq_lens)] if rope_dim else None
    layer = csa2.PagedLayer(nb, rope_dim=rope_dim, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=lat, ropes=ropes)
    q = wl.q_heads(st, 0, B, heads, 512 + rope_dim)
    rng = np.random.default_rng(7)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b, n in enumerate(seq_lens):
        if b == 3:
            continue  # an empty global selection: lse -inf, the window alone
        m = min(n, K)
        idx[b, :m] = rng.choice(n, size=m, replace=False)
    sigma = 1 / math.sqrt(512 + rope_dim)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    out, lse = csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q), to_dev(idx), sigma)
    # the window's own latents (the layer's local KV), positions n-128 .. n-1
    lat_win = [wl.latent_rows(st, 1, b, min(n, 128)) for b, n in enumerate(seq_lens)]
    ring = csa2.SwaRing(B)
    _fill_window(ring, lat_win, seq_lens)
    csa2.csa2_swa_attn_merge(ring, batch.seq_lens, to_dev(q), sigma, out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b, n in enumerate(seq_lens):
        og, lg = oracle_attention_rows(lat[b], ropes[b] if ropes else None, q[b], idx[b], n, sigma)
        codes, scales = oracle.swa.swa_pack(lat_win[b])
        os_, ls = oracle.swa.swa_attention(q[b], oracle.swa.swa_unpack(codes, scales), sigma)
        om, lm = oracle.swa.merge(og, lg, os_, ls)
        err = float(np.max(np.abs(out[b] - om)))
        assert err <= ATTN_TOL, (b, err)
        assert float(np.max(np.abs(lse[b] - lm))) <= LSE_TOL, b


def test_swa_merge_empty_window_leaves_result():
    st = wl.Streams(102)
    ring = csa2.SwaRing(2)
    out = torch.from_numpy(st.gen("misc").standard_normal((2, 16, 512), dtype=np.float32)).cuda()
    lse = torch.from_numpy(np.array([[0.5] * 16, [-np.inf] * 16], dtype=np.float32)).cuda()
    o0, l0 = out.clone(), lse.clone()
    q = to_dev(wl.q_heads(st, 0, 2, 16, 512))
    csa2.csa2_swa_attn_merge(ring, to_dev(np.array([0, -3], dtype=np.int32)), q, 0.05, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o0) and torch.equal(lse, l0)


def _union_case(seed, seq_lens, K, rope_dim, heads, empty_global=(), skip_last=False):
    """A paged layer, a window ring and a selection; returns the GPU inputs and the oracle's union result."""
    st = wl.Streams(seed)
    B = len(seq_lens)
    tables, nb = build_tables(st, seq_lens, True)
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)]
    ropes = [wl.rope_rows(st, 0, b, n, rope_dim) for b, n in enumerate(seq_lens)] if rope_dim else None
    layer = csa2.PagedLayer(nb, rope_dim=rope_dim, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=lat, ropes=ropes)
    q = wl.q_heads(st, 0, B, heads, 512 + rope_dim)
    rng = np.random.default_rng(seed)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b, n in enumerate(seq_lens):
        if b in empty_global:
            continue
        m = min(n, K)
        idx[b, :m] = rng.choice(n, size=m, replace=False)
    sigma = 1 / math.sqrt(512 + rope_dim)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    lat_win = [wl.latent_rows(st, 1, b, min(n, 128)) for b, n in enumerate(seq_lens)]
    ring = csa2.SwaRing(B)
    _fill_window(ring, lat_win, seq_lens, skip_last)
    expect = []
    for b, n in enumerate(seq_lens):
        og, lg = oracle_attention_rows(lat[b], ropes[b] if ropes else None, q[b], idx[b], n, sigma)
        codes, scales = oracle.swa.swa_pack(lat_win[b])
        os_, ls = oracle.swa.swa_attention(q[b], oracle.swa.swa_unpack(codes, scales), sigma)
        expect.append(oracle.swa.merge(og, lg, os_, ls))
    return layer, batch, to_dev(q), to_dev(idx), sigma, ring, expect, lat_win


# (rope_dim, heads, seq_lens, K): batch-1 decode at K 2048 (32 + 4 partials, wide combine) and at the
# decoder's K 512 (16 + 4), mixed lengths
# with windows of 1 .. 128 entries and an empty global selection, 128 heads, a batch of 40 at 128 heads
# (64 heads per workgroup, 2 + 4 partials, the narrow combine) and a batch of 32 with rope at 64 heads per
# workgroup (a ragged last tile of 96 entries)
UNION_CASES = [
    (0, 64, [20000], 2048),
    (0, 64, [70000], 512),
    (0, 64, [1000, 50, 128, 3000, 1], 256),
    (64, 128, [1000, 50, 128, 3000, 1], 256),
    (64, 16, [33, 200, 97], 512),
    (0, 128, [64 + 37 * i for i in range(40)], 64),
    (64, 64, [40 + 53 * i for i in range(32)], 96),
]


@pytest.mark.parametrize("rope_dim,heads,seq_lens,K", UNION_CASES)
def test_attention_with_window_matches_union_attention(rope_dim, heads, seq_lens, K):
    empty = (3,) if len(seq_lens) > 3 else ()
    layer, batch, q, idx, sigma, ring, expect, _ = _union_case(300 + heads + K + rope_dim, seq_lens, K, rope_dim,
                                                               heads, empty_global=empty)
    out, lse = csa2.csa2_sparse_fp4_decode_attn_swa(layer, batch, q, idx, sigma, ring)
    # the two-call path on the same inputs
    out2, lse2 = csa2.csa2_sparse_fp4_decode_attn(layer, batch, q, idx, sigma)
    csa2.csa2_swa_attn_merge(ring, batch.seq_lens, q, sigma, out2, lse2)
    torch.cuda.synchronize()
    out, lse, out2, lse2 = out.cpu().numpy(), lse.cpu().numpy(), out2.cpu().numpy(), lse2.cpu().numpy()
    for b in range(len(seq_lens)):
        om, lm = expect[b]
        err = float(np.max(np.abs(out[b] - om)))
        assert err <= ATTN_TOL, (b, err)
        assert float(np.max(np.abs(lse[b] - lm))) <= LSE_TOL, b
        assert float(np.max(np.abs(out[b] - out2[b]))) <= 2 * ATTN_TOL, b


# Window-only accuracy.  The window's P carries the token scale, so each P is
# a product split into fp16 hi + lo parts; the split keeps P to ~2^-22, which
# puts these outputs within ~1e-5 of the oracle.  A split whose two parts are
# taken from differently rounded copies of the product misses P by one fp16
# ulp of hi (~7e-4 relative) and shows here as errors near 1e-3, so the bound
# is 2e-4 (this case's outputs reach ~60 in magnitude).
WINDOW_ONLY_TOL = 2e-4


@pytest.mark.parametrize("fused", [True, False])
def test_window_only_accuracy(fused):
    heads, K = 128, 64
    seq_lens = [64 + 37 * i for i in range(40)]
    layer, batch, q, idx, sigma, ring, expect, _ = _union_case(492, seq_lens, K, 0, heads,
                                                               empty_global=tuple(range(len(seq_lens))))
    if fused:
        out, lse = csa2.csa2_sparse_fp4_decode_attn_swa(layer, batch, q, idx, sigma, ring)
    else:
        out, lse = csa2.csa2_sparse_fp4_decode_attn(layer, batch, q, idx, sigma)
        csa2.csa2_swa_attn_merge(ring, batch.seq_lens, q, sigma, out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(len(seq_lens)):
        om, lm = expect[b]
        assert float(np.max(np.abs(out[b] - om))) <= WINDOW_ONLY_TOL, b
        assert float(np.max(np.abs(lse[b] - lm))) <= LSE_TOL, b


@pytest.mark.parametrize("rope_dim,heads,seq_lens,K", [(0, 64, [20000], 2048), (64, 16, [33, 200, 97, 128, 1], 512)])
def test_attention_with_window_appends_current_entry(rope_dim, heads, seq_lens, K):
    """The ring holds positions up to n - 2; the call appends position n - 1 and attends over the full window:
    the same result as above, and the ring's new slot equals the standalone pack bit for bit."""
    layer, batch, q, idx, sigma, ring, expect, lat_win = _union_case(400 + heads + K, seq_lens, K, rope_dim, heads,
                                                                     skip_last=True)
    new = np.stack([lw[-1] for lw in lat_win])
    out, lse = csa2.csa2_sparse_fp4_decode_attn_swa(layer, batch, q, idx, sigma, ring, new_latent=to_dev(new))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    codes, scales = ring.codes.cpu().numpy(), ring.scales.cpu().numpy()
    oc, os_ = oracle.swa.swa_pack(new)
    for b, n in enumerate(seq_lens):
        om, lm = expect[b]
        err = float(np.max(np.abs(out[b] - om)))
        assert err <= ATTN_TOL, (b, err)
        assert float(np.max(np.abs(lse[b] - lm))) <= LSE_TOL, b
        slot = int(oracle.swa.window_slot(n - 1))
        assert np.array_equal(codes[b, slot], oc[b]) and scales[b, slot] == os_[b], b
