"""Pins of the oracle's indexer, top-K, hierarchical pool and Reuse.

- top-K against brute-force rank counting on tiny inputs with heavy ties
  (position t is selected iff fewer than K positions beat it, where u beats t
  when its score is larger, or equal with a lower position);
- K >= n selects everything and pads with -1;
- block scores against an explicit loop; the vectorised block max against it;
- the pool against brute force (n = 64, P = 2) and the invariants the
  Hierarchical Sparse Indexer section implies: with n <= 8 P the pool is every
  position and Reindex is plain top-K; with P >= K the Full layer's top-K lies
  in the pool except at exact ties of the K-th score;
- the scores against an fp32-exact case (small integers) and a direct sum;
- the page fact 2048 blocks x 8 positions = 16,384 candidates;
- the multi-head FP4 indexer score (32 heads x 128 dims at the pages' shape):
  exact rational brute force on small integer heads, FP4 keys and dyadic
  weights; per-head ReLU clipping on a hand-computed case; one non-negative
  head reduces to the dot product; invariance under head permutation and
  linearity in the weights; the 72-byte key; Full selection and pool with it
  against rank counting.
"""

import numpy as np

from oracle import indexer


def _rank_select(scores, k):
    n = len(scores)
    sel = set()
    for t in range(n):
        beaten_by = sum(1 for u in range(n) if scores[u] > scores[t] or (scores[u] == scores[t] and u < t))
        if beaten_by < k:
            sel.add(t)
    return sel


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 65))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        for k in range(1, n + 3):
            got = indexer.topk(scores, k)
            valid = set(int(i) for i in got if i >= 0)
            assert valid == _rank_select(scores, k)
            assert np.sum(got < 0) == max(0, k - n)


def test_topk_k_ge_n_selects_all():
    s = np.array([0.5, -1.0, 2.0])
    got = indexer.topk(s, 5)
    assert sorted(got[:3].tolist()) == [0, 1, 2] and got[3:].tolist() == [-1, -1]


def test_scores_exact_small_integers():
    rng = np.random.default_rng(1)
    q = rng.integers(-4, 5, size=64).astype(np.float32)
    k = rng.integers(-4, 5, size=(100, 64)).astype(np.float32)
    s = indexer.index_scores(q, indexer.keys_to_f64(k, "f32"))
    direct = [sum(int(q[d]) * int(k[t, d]) for d in range(64)) for t in range(100)]
    assert s.tolist() == direct


def test_block_scores_loop_vs_vectorised():
    rng = np.random.default_rng(2)
    for n in (1, 7, 8, 9, 63, 64, 65, 1000):
        s = rng.standard_normal(n)
        a = indexer.block_scores(s)
        b = indexer.block_scores_fast(s)
        assert np.array_equal(a, b)
        assert a.shape[0] == -(-n // 8)
        for j in range(a.shape[0]):
            assert a[j] == max(s[8 * j : 8 * j + 8])


def _pool_brute(scores, P, bt=8):
    n = len(scores)
    nb = -(-n // bt)
    bs = [max(scores[j * bt : min(n, j * bt + bt)]) for j in range(nb)]
    return _rank_select(bs, min(P, nb))


def test_pool_brute_force_n64_p2():
    rng = np.random.default_rng(3)
    for trial in range(50):
        scores = rng.integers(-5, 6, size=64).astype(np.float64)
        got = indexer.pool_blocks(scores, 2)
        assert set(int(i) for i in got if i >= 0) == _pool_brute(scores, 2)


def test_pool_covers_all_when_small():
    rng = np.random.default_rng(4)
    n, P = 100, 16  # 13 blocks <= 16
    s = rng.standard_normal(n)
    pool = indexer.pool_blocks(s, P)
    assert sorted(int(i) for i in pool if i >= 0) == list(range(13))
    assert np.array_equal(indexer.pool_positions(pool, n), np.arange(n))
    keys = rng.standard_normal((n, 64))
    q = rng.standard_normal(64).astype(np.float32)
    r = indexer.reindex_select(q, keys, 10, pool)
    f, _ = indexer.full_select(q, keys, 10)
    assert set(r.tolist()) == set(f.tolist())


def test_full_topk_inside_pool_invariant():
    """With P >= K every top-K position lies in a pool block (continuous scores: no ties)."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = int(rng.integers(200, 3000))
        K = int(rng.integers(1, 40))
        P = K + int(rng.integers(0, 5))
        s = rng.standard_normal(n)
        top = indexer.topk(s, K)
        pool = indexer.pool_blocks(s, P)
        pos = set(indexer.pool_positions(pool, n).tolist())
        assert all(int(t) in pos for t in top if t >= 0)


def test_reindex_uses_only_pool_positions():
    rng = np.random.default_rng(6)
    n = 4096
    keys = rng.standard_normal((n, 64))
    q0 = rng.standard_normal(64).astype(np.float32)
    q1 = rng.standard_normal(64).astype(np.float32)
    _, pool = indexer.full_select(q0, keys, 64, pool_blocks_max=32)
    allowed = set(indexer.pool_positions(pool, n).tolist())
    assert len(allowed) == 256
    r = indexer.reindex_select(q1, keys, 64, pool)
    assert all(int(t) in allowed for t in r)
    # brute force over the pool
    s1 = indexer.index_scores(q1, keys)
    ranked = sorted(allowed, key=lambda t: (-s1[t], t))[:64]
    assert set(r.tolist()) == set(ranked)


def test_reuse_is_identity():
    idx = np.array([5, 3, -1])
    out = indexer.reuse_select(idx)
    assert out.tolist() == [5, 3, -1] and out is not idx


def test_pool_size_fact(golden):
    g = golden("kv_facts.json")
    assert g["pool_blocks"]["value"] * g["pool_block_tokens"]["value"] == g["pool_positions"]["value"]


# ---------------------------------------------------------------- multi-head FP4 indexer
def _mh_direct(q, w, k):
    """Brute force with exact rationals: sum_h w[h] * max(0, sum_d q[h, d] k[t, d])."""
    from fractions import Fraction

    out = []
    for t in range(k.shape[0]):
        tot = Fraction(0)
        for h in range(q.shape[0]):
            dot = sum(Fraction(float(q[h, d])) * Fraction(float(k[t, d])) for d in range(q.shape[1]))
            tot += Fraction(float(w[h])) * max(dot, Fraction(0))
        out.append(tot)
    return out


def test_mh_scores_exact_on_small_values():
    """Small integer-valued heads, FP4 keys and dyadic weights: the float64 score is exact."""
    from oracle import fp4

    rng = np.random.default_rng(11)
    H, D, n = 5, 32, 12
    q = rng.integers(-3, 4, size=(H, D)).astype(np.float16)
    w = np.array([0.5, -1.25, 2.0, 0.0, 3.0], dtype=np.float32)
    codes, scales = fp4.fp4_pack(rng.integers(-6, 7, size=(n, D)).astype(np.float32))
    k = indexer.fp4_keys_to_f64(codes, scales)
    got = indexer.index_scores(q, k, w)
    want = _mh_direct(q, w, k)
    assert [float(x) for x in want] == got.tolist()


def test_mh_scores_relu_clips_each_head():
    """A head whose dot is negative adds nothing; the others add w * dot."""
    q = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 2.0]], dtype=np.float16)
    w = np.array([1.0, 10.0, 0.5], dtype=np.float32)
    k = np.array([[3.0, 1.0], [-2.0, -1.0]])
    # t = 0: heads give 3, -3 (clipped), 2 -> 3 + 0 + 1 = 4; t = 1: -2 (clipped), 2, -2 (clipped) -> 20
    assert indexer.index_scores(q, k, w).tolist() == [4.0, 20.0]


def test_mh_scores_single_head_is_the_dot_where_nonnegative():
    rng = np.random.default_rng(12)
    D = 128
    q = rng.integers(0, 3, size=(1, D)).astype(np.float16)
    k = rng.integers(0, 5, size=(40, D)).astype(np.float64)
    assert np.array_equal(indexer.index_scores(q, k, np.ones(1, np.float32)), indexer.index_scores(q[0], k))


def test_mh_scores_head_order_and_weight_scale():
    rng = np.random.default_rng(13)
    H, D = 32, 128
    q = (rng.standard_normal((H, D)) * 4).astype(np.float16)
    w = rng.standard_normal(H).astype(np.float32)
    k = rng.integers(-6, 7, size=(50, D)).astype(np.float64) * 0.5
    perm = rng.permutation(H)
    a = indexer.index_scores(q, k, w)
    np.testing.assert_allclose(indexer.index_scores(q[perm], k, w[perm]), a, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(indexer.index_scores(q, k, 2 * w), 2 * a, rtol=0, atol=0)


def test_fp4_indexer_key_bytes():
    """A 128-dim key in the latent's FP4 format: 64 bytes of nibbles + 8 E4M3 scales."""
    from oracle import fp4

    assert fp4.packed_row_bytes(128) == 72


def test_mh_full_select_brute_force():
    rng = np.random.default_rng(14)
    H, D, n, K = 4, 16, 60, 7
    q = rng.integers(-2, 3, size=(H, D)).astype(np.float16)
    w = np.array([1.0, 0.5, 2.0, 0.25], dtype=np.float32)
    k = rng.integers(-2, 3, size=(n, D)).astype(np.float64)
    idx, pool = indexer.full_select(q, k, K, pool_blocks_max=3, w=w)
    s = [float(x) for x in _mh_direct(q, w, k)]
    assert set(int(i) for i in idx) == _rank_select(s, K)
    bs = indexer.block_scores(s)
    assert set(int(j) for j in pool if j >= 0) == _rank_select(list(bs), 3)
