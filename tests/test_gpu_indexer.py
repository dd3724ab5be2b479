"""GPU parity of indexer scores, exact top-K, Full / hierarchical / Reindex selection."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import build_tables, check_topk, fill_layer, make_batch, to_dev

pytestmark = pytest.mark.gpu


def _keys_layer(seq_lens, dtype, permuted, seed):
    st = wl.Streams(seed)
    tables, nb = build_tables(st, seq_lens, permuted)
    keys = [wl.idx_keys(st, b, n, dtype) for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, idx_dtype=dtype, device="cuda")
    fill_layer(layer, tables, seq_lens, keys=keys)
    return st, tables, keys, layer


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scores_match_oracle(dtype):
    seq_lens = [1000, 64, 1, 4096 + 13]
    st, tables, keys, layer = _keys_layer(seq_lens, dtype, True, 40)
    q = wl.q_idx(st, 0, len(seq_lens))
    max_len = max(seq_lens)
    batch = make_batch(tables, seq_lens, max_len)
    s = csa2.csa2_index_scores(layer, batch, to_dev(q), max_len)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    for b, n in enumerate(seq_lens):
        ref = oracle.indexer.index_scores(q[b], oracle.indexer.keys_to_f64(keys[b], dtype))
        err = np.max(np.abs(s[b, :n] - ref) / (1e-6 + np.abs(ref).max()))
        assert err < 1e-6, (b, err)
        assert np.all(np.isneginf(s[b, n:]))


def test_topk_exact_on_given_scores_with_ties():
    """Integer scores with heavy ties: the index sets must match the oracle exactly."""
    rng = np.random.default_rng(7)
    lens = np.array([0, 1, 37, 300, 2047, 2048, 2049, 5000, 70000], dtype=np.int32)
    M = int(lens.max())
    sc = rng.integers(-20, 21, size=(len(lens), M)).astype(np.float32)
    sc[3, :] = 5.0   # all equal
    sc[5, ::2] = -0.0  # signed zeros must tie with +0
    for K in (1, 7, 256, 2048, 4096):
        idx = csa2.csa2_topk(to_dev(sc), to_dev(lens), K)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(lens):
            ref = oracle.indexer.topk(sc[b, :n].astype(np.float64), K)
            assert set(idx[b].tolist()) == set(ref.tolist()), (K, b)
            assert np.sum(idx[b] < 0) == max(0, K - n)


def test_topk_boundary_pairs_over_a_wide_key_range():
    """Scores spread over [-100, 100] (two histogram levels) with the K-th and (K+1)-th one ulp apart, exactly
    equal (the lower position wins), or three equal values around the K-th (two of them taken): the final
    bin holds two or three items and one or two are taken; the sets must match the oracle exactly."""
    rng = np.random.default_rng(17)
    B, M, K = 6, 5000, 1000
    lens = np.full(B, M, dtype=np.int32)
    sc = rng.uniform(-100.0, 100.0, size=(B, M)).astype(np.float32)
    for b in range(B):
        order = np.argsort(-sc[b].astype(np.float64), kind="stable")
        kth, nxt, prv = order[K - 1], order[K], order[K - 2]
        if b % 3 == 0:    # one ulp below the K-th
            sc[b, nxt] = np.nextafter(sc[b, kth], np.float32(-np.inf))
        elif b % 3 == 1:  # equal to the K-th, at a lower or a higher position
            sc[b, nxt] = sc[b, kth]
        else:             # three equal values around the K-th
            sc[b, nxt] = sc[b, kth]
            sc[b, prv] = sc[b, kth]
    idx = csa2.csa2_topk(to_dev(sc), to_dev(lens), K)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for b in range(B):
        ref = oracle.indexer.topk(sc[b].astype(np.float64), K)
        assert set(idx[b].tolist()) == set(ref.tolist()), b


def test_topk_narrow_key_range():
    """Scores within a few thousand ulps of each other: the histogram bins are single keys, so
    a partly taken bin is a group of equal scores ranked by position."""
    rng = np.random.default_rng(9)
    lens = np.array([37, 64, 65, 2, 5000], dtype=np.int32)
    M = int(lens.max())
    ulps = rng.integers(0, 40, size=(len(lens), M)).astype(np.int64)
    sc = (np.float32(1.5).view(np.int32) + ulps).astype(np.int32).view(np.float32)
    sc[0, :] = np.float32(-3.25)  # one value
    for K in (1, 7, 33, 2048):
        idx = csa2.csa2_topk(to_dev(sc), to_dev(lens), K)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(lens):
            ref = oracle.indexer.topk(sc[b, :n].astype(np.float64), K)
            assert set(idx[b].tolist()) == set(ref.tolist()), (K, b)


def test_topk_random_scores_repeatable_workspace():
    rng = np.random.default_rng(8)
    lens = np.array([65536, 30000, 4096], dtype=np.int32)
    sc = rng.standard_normal((3, 65536)).astype(np.float32)
    ws = csa2.workspace(csa2.topk_workspace_bytes(3, 65536, 2048))
    for rep in range(3):  # the workspace is left zeroed by each call
        idx = csa2.csa2_topk(to_dev(sc), to_dev(lens), 2048, ws=ws)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(lens):
            ref = oracle.indexer.topk(sc[b, :n].astype(np.float64), 2048)
            assert set(idx[b].tolist()) == set(ref.tolist()), (rep, b)


@pytest.mark.parametrize("dtype,permuted", [("f32", False), ("bf16", True)])
def test_full_select(dtype, permuted):
    seq_lens = [4096, 65536 + 17, 100, 3000]
    st, tables, keys, layer = _keys_layer(seq_lens, dtype, permuted, 41)
    q = wl.q_idx(st, 0, len(seq_lens))
    batch = make_batch(tables, seq_lens, max(seq_lens))
    for K in (256, 512, 2048):
        idx, _ = csa2.csa2_index_select(layer, batch, to_dev(q), K, csa2.FULL)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(seq_lens):
            s = oracle.indexer.index_scores(q[b], oracle.indexer.keys_to_f64(keys[b], dtype))
            check_topk(idx[b], dict(enumerate(s)), K, where=f"K={K} b={b}")


@pytest.mark.parametrize("K", [512, 2048])
def test_hierarchical_pool_and_reindex(K):
    seq_lens = [200000, 16384, 50, 70001]
    P = 2048
    st, tables, keys, layer = _keys_layer(seq_lens, "bf16", True, 42)
    q0 = wl.q_idx(st, 0, len(seq_lens))
    q1 = wl.q_idx(st, 1, len(seq_lens))
    batch = make_batch(tables, seq_lens, max(seq_lens))
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q0), K, csa2.FULL, pool_blocks=P, want_pool=True)
    torch.cuda.synchronize()
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    # Reindex stage fed with the oracle's pool, so a difference is the Reindex kernel's
    o_pools = []
    for b, n in enumerate(seq_lens):
        kf = oracle.indexer.keys_to_f64(keys[b], "bf16")
        s0 = oracle.indexer.index_scores(q0[b], kf)
        bs = oracle.indexer.block_scores_fast(s0)
        nb = len(bs)
        check_topk(pool[b], dict(enumerate(bs)), P, where=f"pool b={b}")
        check_topk(idx[b], dict(enumerate(s0)), K, where=f"full b={b}")
        o_pools.append(oracle.indexer.pool_blocks(s0, P))
        assert np.sum(pool[b] >= 0) == min(P, nb)
    o_pool_t = to_dev(np.stack(o_pools).astype(np.int32))
    idx1, _ = csa2.csa2_index_select(layer, batch, to_dev(q1), K, csa2.REINDEX, pool_in=o_pool_t, pool_blocks=P)
    torch.cuda.synchronize()
    idx1 = idx1.cpu().numpy()
    for b, n in enumerate(seq_lens):
        kf = oracle.indexer.keys_to_f64(keys[b], "bf16")
        pos = oracle.indexer.pool_positions(o_pools[b], n)
        s1 = oracle.indexer.index_scores(q1[b], kf[pos])
        check_topk(idx1[b], dict(zip(pos.tolist(), s1)), K, where=f"reindex b={b}")


def test_select_rejects_bad_args():
    seq_lens = [64]
    st, tables, keys, layer = _keys_layer(seq_lens, "bf16", False, 43)
    batch = make_batch(tables, seq_lens, 64)
    q = to_dev(wl.q_idx(st, 0, 1))
    with pytest.raises(csa2.Csa2Error):
        csa2.csa2_index_select(layer, batch, q, 0, csa2.FULL)
    with pytest.raises(csa2.Csa2Error):  # pool larger than 2048 blocks
        csa2.csa2_index_select(layer, batch, q, 64, csa2.FULL, pool_blocks=4096, want_pool=True)


def test_topk_clustered_scores_take_the_exact_fallback():
    """Monotone scores put the whole top-K in the last segments, which overflows the
    per-segment candidate budget; the select must fall back and stay exact."""
    lens = np.array([200000, 100000, 5000], dtype=np.int32)
    M = int(lens.max())
    sc = np.tile(np.arange(M, dtype=np.float32), (3, 1))
    sc[1] = -sc[1]  # top-K at the front
    sc[2, :] = np.float32(1.0)
    sc[2, 1000:3000] = 2.0
    for K in (64, 2048, 4096):
        idx = csa2.csa2_topk(to_dev(sc), to_dev(lens), K)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(lens):
            ref = oracle.indexer.topk(sc[b, :n].astype(np.float64), K)
            assert idx[b].tolist() == sorted(ref.tolist(), key=lambda v: (v < 0, v)), (K, b)


def _clustered_keys_layer(n, q, lo, hi, seed):
    """bf16 keys whose scores against q are large exactly on positions [lo, hi)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, 64)).astype(np.float32)
    k[lo:hi] += 8.0 * q[None, :] / np.linalg.norm(q)
    keys = wl.to_bf16_bits(k)
    tables = np.arange(-(-n // 64), dtype=np.int32)[None]
    layer = csa2.PagedLayer(tables.shape[1], idx_dtype="bf16", device="cuda")
    fill_layer(layer, tables, [n], keys=[keys])
    return keys, tables, layer


@pytest.mark.parametrize("hier", [False, True])
def test_full_select_clustered_scores(hier):
    n = 300000
    q = np.random.default_rng(5).standard_normal(64).astype(np.float32)
    keys, tables, layer = _clustered_keys_layer(n, q, 123456, 123456 + 9000, 6)
    batch = make_batch(tables, [n], n)
    K, P = 2048, 2048
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q[None]), K, csa2.FULL, pool_blocks=P, want_pool=hier)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()[0]
    s = oracle.indexer.index_scores(q, oracle.indexer.keys_to_f64(keys, "bf16"))
    check_topk(idx, dict(enumerate(s)), K, where="clustered full")
    assert np.all(np.diff(idx[idx >= 0]) > 0), "indices are written in increasing order"
    if hier:
        pool = pool.cpu().numpy()[0]
        check_topk(pool, dict(enumerate(oracle.indexer.block_scores_fast(s))), P, where="clustered pool")
        assert np.all(np.diff(pool[pool >= 0]) > 0)


def test_select_is_deterministic():
    seq_lens = [70000, 9000]
    st, tables, keys, layer = _keys_layer(seq_lens, "bf16", True, 44)
    q = to_dev(wl.q_idx(st, 0, 2))
    batch = make_batch(tables, seq_lens, 70000)
    a, pa = csa2.csa2_index_select(layer, batch, q, 2048, csa2.FULL, pool_blocks=2048, want_pool=True)
    b, pb = csa2.csa2_index_select(layer, batch, q, 2048, csa2.FULL, pool_blocks=2048, want_pool=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(pa, pb)


def test_full_select_1m_hierarchical_and_reindex():
    """The 1M-token shape: 512 scan segments with small candidate budgets (top-12 extraction per segment)."""
    seq_lens = [1 << 20, 700001]
    P, K = 2048, 2048
    st, tables, keys, layer = _keys_layer(seq_lens, "bf16", False, 45)
    q0 = wl.q_idx(st, 0, len(seq_lens))
    q1 = wl.q_idx(st, 1, len(seq_lens))
    batch = make_batch(tables, seq_lens, max(seq_lens))
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q0), K, csa2.FULL, pool_blocks=P, want_pool=True)
    idx1, _ = csa2.csa2_index_select(layer, batch, to_dev(q1), K, csa2.REINDEX, pool_in=pool, pool_blocks=P)
    torch.cuda.synchronize()
    idx, pool, idx1 = idx.cpu().numpy(), pool.cpu().numpy(), idx1.cpu().numpy()
    for b, n in enumerate(seq_lens):
        kf = oracle.indexer.keys_to_f64(keys[b], "bf16")
        s0 = oracle.indexer.index_scores(q0[b], kf)
        check_topk(idx[b], dict(enumerate(s0)), K, where=f"1M full b={b}")
        assert np.all(np.diff(idx[b][idx[b] >= 0]) > 0)
        check_topk(pool[b], dict(enumerate(oracle.indexer.block_scores_fast(s0))), P, where=f"1M pool b={b}")
        # Reindex over the GPU's pool: every pool block is a valid block, so score its positions
        pos = oracle.indexer.pool_positions(pool[b][pool[b] >= 0], n)
        s1 = oracle.indexer.index_scores(q1[b], kf[pos])
        check_topk(idx1[b], dict(zip(pos.tolist(), s1)), K, where=f"1M reindex b={b}")


def test_full_select_1m_heavy_ties():
    """Integer-valued keys and query: scores tie in large groups at the K-th value, so segment
    cuts fall inside ties and the select must re-read segments (or run over every stored key)."""
    n = 1 << 20
    rng = np.random.default_rng(46)
    k = rng.integers(-2, 3, size=(n, 64)).astype(np.float32)
    keys = wl.to_bf16_bits(k)
    q = np.zeros((1, 64), dtype=np.float32)
    q[0, :4] = 1.0
    tables = np.arange(n // 64, dtype=np.int32)[None]
    layer = csa2.PagedLayer(tables.shape[1], idx_dtype="bf16", device="cuda")
    fill_layer(layer, tables, [n], keys=[keys])
    batch = make_batch(tables, [n], n)
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q), 2048, csa2.FULL, pool_blocks=2048, want_pool=True)
    torch.cuda.synchronize()
    idx, pool = idx.cpu().numpy()[0], pool.cpu().numpy()[0]
    s = oracle.indexer.index_scores(q[0], oracle.indexer.keys_to_f64(keys, "bf16"))
    ref = oracle.indexer.topk(s, 2048)
    assert set(idx.tolist()) == set(ref.tolist()), "exact ties: lower positions win"
    bs = oracle.indexer.block_scores_fast(s)
    assert set(pool.tolist()) == set(oracle.indexer.topk(bs, 2048).tolist())


# ---------------------------------------------------------------- multi-head FP4 indexer keys
def _fp4_layer(seq_lens, heads, permuted, seed):
    st = wl.Streams(seed)
    tables, nb = build_tables(st, seq_lens, permuted)
    keys = [wl.idx4_keys(st, b, n) for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, idx_dtype="fp4", idx_heads=heads, device="cuda")
    fill_layer(layer, tables, seq_lens, keys=keys)
    return st, tables, keys, layer


def _fp4_oracle_keys(layer, tables, keys, b, n, check_stored=True):
    """Oracle float64 keys of sequence b (packed by the oracle), and the stored bytes compared bit-exact."""
    if n > (1 << 18):  # the oracle's pack in slices (memory)
        parts = [oracle.fp4.fp4_pack(keys[b][s:s + (1 << 18)]) for s in range(0, n, 1 << 18)]
        codes, scales = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    else:
        codes, scales = oracle.fp4.fp4_pack(keys[b])
    if check_stored and n:
        rows = torch.from_numpy(oracle.paged.physical_rows(tables[b], np.arange(n))).cuda()
        assert np.array_equal(layer.idx_keys[rows].cpu().numpy(), codes), f"stored codes b={b}"
        assert np.array_equal(layer.idx_scales[rows].cpu().numpy(), scales), f"stored scales b={b}"
    return oracle.indexer.fp4_keys_to_f64(codes, scales)


@pytest.mark.parametrize("heads", [32, 7, 1])
def test_fp4_scores_match_oracle(heads):
    seq_lens = [1000, 64, 1, 4096 + 13, 0]
    st, tables, keys, layer = _fp4_layer(seq_lens, heads, True, 50)
    q = wl.q_idx_heads(st, 0, len(seq_lens), heads)
    w = wl.w_idx(st, 0, len(seq_lens), heads)
    max_len = max(seq_lens) + 5
    batch = make_batch(tables, seq_lens, max_len)
    s = csa2.csa2_index_scores(layer, batch, to_dev(q), max_len, w_idx=to_dev(w))
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    for b, n in enumerate(seq_lens):
        kf = _fp4_oracle_keys(layer, tables, keys, b, n)
        ref = oracle.indexer.index_scores(q[b], kf, w[b])
        # fp32 accumulation: error bounded by a few ulps of the sum of absolute terms
        mag = np.maximum(np.abs(kf) @ np.abs(q[b].astype(np.float64)).T, 0.0) @ np.abs(w[b].astype(np.float64))
        err = np.abs(s[b, :n] - ref)
        assert np.all(err <= 1e-6 * mag + 1e-30), (b, float(np.max(err / (mag + 1e-30))))
        assert np.all(np.isneginf(s[b, n:]))


@pytest.mark.parametrize("permuted", [False, True])
def test_fp4_full_select(permuted):
    seq_lens = [4096, 65536 + 17, 100, 3000]
    st, tables, keys, layer = _fp4_layer(seq_lens, 32, permuted, 51)
    q, w = wl.q_idx_heads(st, 0, len(seq_lens)), wl.w_idx(st, 0, len(seq_lens))
    batch = make_batch(tables, seq_lens, max(seq_lens))
    for K in (256, 512, 2048):
        idx, _ = csa2.csa2_index_select(layer, batch, to_dev(q), K, csa2.FULL, w_idx=to_dev(w))
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        for b, n in enumerate(seq_lens):
            s = oracle.indexer.index_scores(q[b], _fp4_oracle_keys(layer, tables, keys, b, n, K == 256), w[b])
            check_topk(idx[b], dict(enumerate(s)), K, where=f"K={K} b={b}")


@pytest.mark.parametrize("K", [512, 2048])
def test_fp4_hierarchical_pool_and_reindex(K):
    seq_lens = [200000, 16384, 50, 70001]
    P = 2048
    st, tables, keys, layer = _fp4_layer(seq_lens, 32, True, 52)
    q0, w0 = wl.q_idx_heads(st, 0, len(seq_lens)), wl.w_idx(st, 0, len(seq_lens))
    q1, w1 = wl.q_idx_heads(st, 1, len(seq_lens)), wl.w_idx(st, 1, len(seq_lens))
    batch = make_batch(tables, seq_lens, max(seq_lens))
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q0), K, csa2.FULL, pool_blocks=P, want_pool=True,
                                       w_idx=to_dev(w0))
    torch.cuda.synchronize()
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    o_pools, kfs = [], []
    for b, n in enumerate(seq_lens):
        kf = _fp4_oracle_keys(layer, tables, keys, b, n)
        kfs.append(kf)
        s0 = oracle.indexer.index_scores(q0[b], kf, w0[b])
        check_topk(pool[b], dict(enumerate(oracle.indexer.block_scores_fast(s0))), P, where=f"pool b={b}")
        check_topk(idx[b], dict(enumerate(s0)), K, where=f"full b={b}")
        o_pools.append(oracle.indexer.pool_blocks(s0, P))
    # Reindex fed with the oracle's pool, so a difference is the Reindex kernel's
    o_pool_t = to_dev(np.stack(o_pools).astype(np.int32))
    idx1, _ = csa2.csa2_index_select(layer, batch, to_dev(q1), K, csa2.REINDEX, pool_in=o_pool_t, pool_blocks=P,
                                     w_idx=to_dev(w1))
    torch.cuda.synchronize()
    idx1 = idx1.cpu().numpy()
    for b, n in enumerate(seq_lens):
        pos = oracle.indexer.pool_positions(o_pools[b], n)
        s1 = oracle.indexer.index_scores(q1[b], kfs[b][pos], w1[b])
        check_topk(idx1[b], dict(zip(pos.tolist(), s1)), K, where=f"reindex b={b}")


def test_fp4_append_packs_keys():
    """kv_append stores a 128-dim fp32 key as FP4 codes + E4M3 scales, bit-exact with the oracle's pack,
    at the physical slot of position seq_lens[b] and nowhere else."""
    st = wl.Streams(53)
    seq_lens = [63, 64, 0, 130]
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    layer = csa2.PagedLayer(nb, idx_dtype="fp4", device="cuda")
    batch = make_batch(tables, seq_lens)
    new_keys = wl.idx4_keys(st, 99, len(seq_lens))
    new_keys[1, :16] = 0.0     # an all-zero group
    new_keys[2, 16:32] *= 1e4  # a group whose scale saturates
    csa2.csa2_kv_append(layer, batch, None, None, to_dev(new_keys))
    torch.cuda.synchronize()
    codes, scales = oracle.fp4.fp4_pack(new_keys)
    gc, gs = layer.idx_keys.cpu().numpy(), layer.idx_scales.cpu().numpy()
    written = []
    for b, n in enumerate(seq_lens):
        row = int(oracle.paged.physical_rows(tables[b], np.array([n]))[0])
        written.append(row)
        assert np.array_equal(gc[row], codes[b]) and np.array_equal(gs[row], scales[b]), b
    others = np.setdiff1d(np.arange(gc.shape[0]), written)
    assert not gc[others].any() and not gs[others].any()


@pytest.mark.parametrize("K", [512])
def test_fp4_full_select_1m_hierarchical_and_reindex(K):
    """The decoder's indexer at full size: 1,048,576 FP4 keys of 128 dims, 32 weighted heads, top-K 512, the
    2048 x 8 pool and a Reindex over it (the launch shapes the 1M benchmarks time)."""
    n = 1 << 20
    P = 2048
    st, tables, keys, layer = _fp4_layer([n], 32, False, 54)
    q0, w0 = wl.q_idx_heads(st, 0, 1), wl.w_idx(st, 0, 1)
    q1, w1 = wl.q_idx_heads(st, 1, 1), wl.w_idx(st, 1, 1)
    batch = make_batch(tables, [n], n)
    idx, pool = csa2.csa2_index_select(layer, batch, to_dev(q0), K, csa2.FULL, pool_blocks=P, want_pool=True,
                                       w_idx=to_dev(w0))
    idx1, _ = csa2.csa2_index_select(layer, batch, to_dev(q1), K, csa2.REINDEX, pool_in=pool, pool_blocks=P,
                                     w_idx=to_dev(w1))
    torch.cuda.synchronize()
    idx, pool, idx1 = idx.cpu().numpy()[0], pool.cpu().numpy()[0], idx1.cpu().numpy()[0]
    kf = _fp4_oracle_keys(layer, tables, keys, 0, n, check_stored=False)
    s0 = oracle.indexer.index_scores(q0[0], kf, w0[0])
    check_topk(idx, dict(enumerate(s0)), K, where="1M fp4 full")
    assert np.all(np.diff(idx[idx >= 0]) > 0)
    check_topk(pool, dict(enumerate(oracle.indexer.block_scores_fast(s0))), P, where="1M fp4 pool")
    pos = oracle.indexer.pool_positions(pool[pool >= 0], n)
    s1 = oracle.indexer.index_scores(q1[0], kf[pos], w1[0])
    check_topk(idx1, dict(zip(pos.tolist(), s1)), K, where="1M fp4 reindex")
