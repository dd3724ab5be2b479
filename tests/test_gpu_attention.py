"""GPU parity of sparse FP4 decode attention (max abs error <= 2e-3 vs the oracle)."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import ATTN_TOL, LSE_TOL, build_tables, fill_layer, make_batch, oracle_attention_rows, to_dev

pytestmark = pytest.mark.gpu


def _setup(seq_lens, heads, rope_dim, permuted, seed):
    st = wl.Streams(seed)
    tables, nb = build_tables(st, seq_lens, permuted)
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)]
    ropes = [wl.rope_rows(st, 0, b, n, rope_dim) for b, n in enumerate(seq_lens)] if rope_dim else None
    layer = csa2.PagedLayer(nb, rope_dim=rope_dim, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=lat, ropes=ropes)
    q = wl.q_heads(st, 0, len(seq_lens), heads, 512 + rope_dim)
    return st, tables, lat, ropes, layer, q


def _run_and_check(seq_lens, heads, K, rope_dim=0, permuted=True, seed=50, idx=None, sigma=None):
    st, tables, lat, ropes, layer, q = _setup(seq_lens, heads, rope_dim, permuted, seed)
    B = len(seq_lens)
    rng = np.random.default_rng(seed)
    if idx is None:
        idx = np.full((B, K), -1, dtype=np.int32)
        for b, n in enumerate(seq_lens):
            m = min(n, K)
            idx[b, :m] = rng.choice(n, size=m, replace=False)
    sigma = sigma or 1 / math.sqrt(512 + rope_dim)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    out, lse = csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q), to_dev(idx), sigma)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for b, n in enumerate(seq_lens):
        o_out, o_lse = oracle_attention_rows(lat[b], ropes[b] if ropes else None, q[b], idx[b], n, sigma)
        err = float(np.max(np.abs(out[b] - o_out)))
        worst = max(worst, err)
        assert err <= ATTN_TOL, (b, err)
        fin = np.isfinite(o_lse)
        assert np.array_equal(fin, np.isfinite(lse[b]))
        if fin.any():
            assert np.max(np.abs(lse[b][fin] - o_lse[fin])) <= LSE_TOL
    return worst


def test_config1_shape():
    _run_and_check([4096], 16, 256, permuted=False)


def test_rope_batch_permuted():
    _run_and_check([5000, 70000, 2048], 64, 2048, rope_dim=64)


@pytest.mark.parametrize("heads", [16, 32, 48, 64, 128])
def test_head_counts(heads):
    _run_and_check([3000, 777], heads, 300)


@pytest.mark.parametrize("K", [1, 31, 33, 1000, 4096])
def test_ragged_topk(K):
    _run_and_check([6000], 64, K)


def test_decoder_topk512():
    """The decoder's top-K of 512 entries, 64 heads, long sequences."""
    _run_and_check([65536, 100000], 64, 512, seed=53)


def test_invalid_and_empty_selections():
    seq_lens = [500, 10, 300]
    K = 64
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 500, size=(3, K)).astype(np.int32)
    idx[0, :4] = [-1, -5, 500, 10000]
    idx[1] = -1  # nothing selected -> out 0, lse -inf
    idx[2, ::3] = 299
    idx[2, 1::3] = 300  # == length: skipped
    # duplicates are allowed in the kernel's input and count twice, like the oracle
    _run_and_check(seq_lens, 64, K, idx=idx)


def test_outlier_stress_small_sigma_and_large_sigma():
    _run_and_check([8192], 64, 2048, sigma=0.2)
    _run_and_check([8192], 64, 2048, sigma=0.001)


def test_identity_vs_permuted_table_bitwise():
    """Same logical cache, different physical layout -> identical bits (paged addressing)."""
    seq_lens = [3000, 4100]
    outs = []
    for permuted in (False, True):
        st = wl.Streams(60)
        tables, nb = build_tables(st, seq_lens, permuted)
        st2 = wl.Streams(61)
        lat = [wl.latent_rows(st2, 0, b, n) for b, n in enumerate(seq_lens)]
        layer = csa2.PagedLayer(nb, device="cuda")
        fill_layer(layer, tables, seq_lens, latents=lat)
        q = wl.q_heads(st2, 0, 2, 64, 512)
        idx = np.stack([np.random.default_rng(b).choice(n, 1024, replace=False) for b, n in enumerate(seq_lens)])
        out, lse = csa2.csa2_sparse_fp4_decode_attn(layer, make_batch(tables, seq_lens, 4100), to_dev(q),
                                                    to_dev(idx.astype(np.int32)), 1 / math.sqrt(512))
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_batch8_64k_rope_launch_shape():
    """8 sequences x 65,536 tokens, 64 heads + rope, K 2048: the 32-heads-per-workgroup split launch of batched
    decode."""
    _run_and_check([65536] * 8, 64, 2048, rope_dim=64, seed=51)


def test_batch32_launch_shape():
    """32 sequences, 64 heads, K 2048: the 64-heads-per-workgroup launch used for large batches."""
    rng = np.random.default_rng(52)
    lens = [int(v) for v in np.exp(rng.uniform(np.log(1500), np.log(40000), size=32))]
    _run_and_check(lens, 64, 2048, seed=52)


def test_attention_1m_decoder_shape():
    """The decoder's attention at full size: one sequence of 1,048,576 positions behind a permuted page
    table, 64 heads, top-K 512.  Only the selected rows are filled (with their own latents); any read of
    another row would see zeros and fail the comparison."""
    n, H, K = 1 << 20, 64, 512
    st = wl.Streams(55)
    tables, nb = build_tables(st, [n], True)
    rng = np.random.default_rng(55)
    sel = np.sort(rng.choice(n, size=K, replace=False)).astype(np.int32)
    lat_sel = wl.latent_rows(st, 0, 0, K)
    layer = csa2.PagedLayer(nb, device="cuda")
    rows = torch.from_numpy(oracle.paged.physical_rows(tables[0], sel)).cuda()
    codes, scales = csa2.csa2_fp4_pack(to_dev(lat_sel))
    layer.codes[rows] = codes
    layer.scales[rows] = scales
    q = wl.q_heads(st, 0, 1, H, 512)
    sigma = 1 / math.sqrt(512)
    batch = make_batch(tables, [n], n)
    out, lse = csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q), to_dev(sel[None]), sigma)
    torch.cuda.synchronize()
    c = oracle.fp4.fp4_unpack(*oracle.fp4.fp4_pack(lat_sel))
    o_out, o_lse = oracle.attention.sparse_attention(q[0], c, sigma)
    assert float(np.max(np.abs(out.cpu().numpy()[0] - o_out))) <= ATTN_TOL
    assert float(np.max(np.abs(lse.cpu().numpy()[0] - o_lse))) <= LSE_TOL
