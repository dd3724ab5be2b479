"""GPU parity of the multi-layer entry points: several layers' attention in one launch, several Reindex
layers in one pool-scoring and one select launch, and a Full selection with this step's appends riding in
the scan's launch.  Each is checked against the oracle and against the single-layer calls it stands for."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import (ATTN_TOL, LSE_TOL, build_tables, check_topk, fill_layer, make_batch, oracle_attention_rows,
                   to_dev)

pytestmark = pytest.mark.gpu


def _random_idx(rng, seq_lens, K):
    idx = np.full((len(seq_lens), K), -1, dtype=np.int32)
    for b, n in enumerate(seq_lens):
        m = min(n, K)
        idx[b, :m] = rng.choice(n, size=m, replace=False)
    return idx


@pytest.mark.parametrize("seq_lens,K,heads,rope_dim", [
    ([20000], 2048, 64, 0),                 # batch-1 decode: four layers share the launch (16 splits each)
    ([5000, 700, 33000], 512, 64, 0),       # ragged batch at the decoder's top-K
    ([3000, 4100], 300, 64, 64),            # rope side-band
    ([64 + 37 * i for i in range(40)], 64, 128, 0),  # many sequences, 64 heads per workgroup
])
def test_attention_layers_own_kv(seq_lens, K, heads, rope_dim):
    """Four layers, each with its own KV pool (Reuse: layers 0 and 1 share one index set, 2 and 3 have their
    own): every layer matches the oracle over its own cache, and the single-layer call within 5e-5."""
    st = wl.Streams(700 + K + heads + rope_dim)
    B, L = len(seq_lens), 4
    tables, nb = build_tables(st, seq_lens, True)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    lat = [[wl.latent_rows(st, l, b, n) for b, n in enumerate(seq_lens)] for l in range(L)]
    ropes = [[wl.rope_rows(st, l, b, n, rope_dim) for b, n in enumerate(seq_lens)] if rope_dim else None
             for l in range(L)]
    layers = []
    for l in range(L):
        layer = csa2.PagedLayer(nb, rope_dim=rope_dim, device="cuda")
        fill_layer(layer, tables, seq_lens, latents=lat[l], ropes=ropes[l])
        layers.append(layer)
    q = [wl.q_heads(st, l, B, heads, 512 + rope_dim) for l in range(L)]
    rng = np.random.default_rng(K)
    shared = _random_idx(rng, seq_lens, K)
    idx = [shared, shared, _random_idx(rng, seq_lens, K), _random_idx(rng, seq_lens, K)]
    sigma = 1 / math.sqrt(512 + rope_dim)
    jobs = [(layers[l], to_dev(q[l]), to_dev(idx[l])) for l in range(L)]
    outs, lses = csa2.csa2_sparse_fp4_decode_attn_layers(jobs, batch, sigma)
    singles = [csa2.csa2_sparse_fp4_decode_attn(layers[l], batch, jobs[l][1], jobs[l][2], sigma) for l in range(L)]
    torch.cuda.synchronize()
    for l in range(L):
        out, lse = outs[l].cpu().numpy(), lses[l].cpu().numpy()
        o1, l1 = singles[l][0].cpu().numpy(), singles[l][1].cpu().numpy()
        # the launch holds more problems, so its entries are split differently and its heads may be grouped
        # differently (64, 32 or 16 per workgroup: each logit's channel sum in 2 or 4 fp32 partials); each result
        # is within ~2e-5 of the exact one, so the two differ by the rounding of both
        assert np.all(np.abs(out - o1) <= 5e-5 * np.maximum(1.0, np.abs(o1))), l
        for b, n in enumerate(seq_lens):
            o_out, o_lse = oracle_attention_rows(lat[l][b], ropes[l][b] if rope_dim else None, q[l][b], idx[l][b], n,
                                                 sigma)
            assert float(np.max(np.abs(out[b] - o_out))) <= ATTN_TOL, (l, b)
            assert float(np.max(np.abs(lse[b] - o_lse))) <= LSE_TOL, (l, b)


def test_attention_layers_with_windows():
    """Three layers, each with its own sliding-window ring and new window entry, in one launch: the same as
    one csa2_sparse_fp4_decode_attn_swa call per layer (within 5e-5: the launch of 9 problems groups 32 heads
    per workgroup, the single calls 16), and the same ring bytes."""
    st = wl.Streams(720)
    seq_lens, K, H, L = [3000, 90, 128], 256, 64, 3
    B = len(seq_lens)
    tables, nb = build_tables(st, seq_lens, True)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    layer = csa2.PagedLayer(nb, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=[wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)])
    rng = np.random.default_rng(5)
    idx = to_dev(_random_idx(rng, seq_lens, K))
    sigma = 1 / math.sqrt(512)
    rings_a, rings_b, new = [], [], []
    for l in range(L):
        ra, rb = csa2.SwaRing(B), csa2.SwaRing(B)
        for j in range(128):  # fill every slot, then append the last position again as the new entry
            pos = np.array([n - min(n, 128) + j if j < min(n, 128) else -1 for n in seq_lens], dtype=np.int32)
            rows = to_dev(wl.latent_rows(st, 10 + l, j, B))
            csa2.csa2_swa_append(ra, to_dev(pos), rows)
            csa2.csa2_swa_append(rb, to_dev(pos), rows)
        rings_a.append(ra)
        rings_b.append(rb)
        new.append(to_dev(wl.latent_rows(st, 20 + l, 0, B)))
    q = [to_dev(wl.q_heads(st, l, B, H, 512)) for l in range(L)]
    outs, lses = csa2.csa2_sparse_fp4_decode_attn_layers(
        [(layer, q[l], idx, rings_a[l], new[l]) for l in range(L)], batch, sigma)
    singles = [csa2.csa2_sparse_fp4_decode_attn_swa(layer, batch, q[l], idx, sigma, rings_b[l], new_latent=new[l])
               for l in range(L)]
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.equal(rings_a[l].codes, rings_b[l].codes) and torch.equal(rings_a[l].scales, rings_b[l].scales)
        o1 = singles[l][0]
        assert bool(((outs[l] - o1).abs() <= 5e-5 * o1.abs().clamp(min=1.0)).all())
        assert float((lses[l] - singles[l][1]).abs().max()) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp4"])
def test_reindex_layers_equal_single_calls(dtype):
    """Three Reindex layers over one Full layer's pool in two launches: indices identical to one
    csa2_index_select REINDEX call per layer (same kernels, deterministic), and exact against the oracle."""
    st = wl.Streams(730)
    seq_lens, K, P = [40000, 3000, 17], 512, 2048
    B = len(seq_lens)
    tables, nb = build_tables(st, seq_lens, True)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    fp4 = dtype == "fp4"
    keys = [wl.idx4_keys(st, b, n) if fp4 else wl.idx_keys(st, b, n, dtype) for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, idx_dtype=dtype, device="cuda")
    fill_layer(layer, tables, seq_lens, keys=keys)
    if fp4:
        qs = [(to_dev(wl.q_idx_heads(st, l, B)), to_dev(wl.w_idx(st, l, B))) for l in range(4)]
    else:
        qs = [(to_dev(wl.q_idx(st, l, B)), None) for l in range(4)]
    _, pool = csa2.csa2_index_select(layer, batch, qs[0][0], K, csa2.FULL, pool_blocks=P, want_pool=True,
                                     w_idx=qs[0][1])
    multi = csa2.csa2_index_reindex_layers(layer, batch, qs[1:], K, pool, P)
    single = [csa2.csa2_index_select(layer, batch, q, K, csa2.REINDEX, pool_in=pool, pool_blocks=P, w_idx=w)[0]
              for q, w in qs[1:]]
    torch.cuda.synchronize()
    pool = pool.cpu().numpy()
    for l in range(3):
        assert torch.equal(multi[l], single[l]), l
        got = multi[l].cpu().numpy()
        for b, n in enumerate(seq_lens):
            kf = (oracle.indexer.fp4_keys_to_f64(*oracle.fp4.fp4_pack(keys[b])) if fp4
                  else oracle.indexer.keys_to_f64(keys[b], dtype))
            pos = oracle.indexer.pool_positions(pool[b][pool[b] >= 0], n)
            q, w = (x.cpu().numpy()[b] if x is not None else None for x in qs[l + 1])
            s = oracle.indexer.index_scores(q, kf[pos], w) if fp4 else oracle.indexer.index_scores(q, kf[pos])
            check_topk(got[b], dict(zip(pos.tolist(), s)), K, where=f"reindex layer {l} b={b}")


def _append_case(dtype, seq_lens_new, seed):
    """Caches holding positions 0 .. n - 2 and the inputs of the row at n - 1, twice (one per path)."""
    st = wl.Streams(seed)
    fp4 = dtype == "fp4"
    tables, nb = build_tables(st, seq_lens_new, True, extra_blocks=1)
    old = [n - 1 for n in seq_lens_new]
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens_new)]
    keys = [wl.idx4_keys(st, b, n) if fp4 else wl.idx_keys(st, b, n, dtype) for b, n in enumerate(seq_lens_new)]
    pair = []
    for _ in range(2):
        layer = csa2.PagedLayer(nb, idx_dtype=dtype, device="cuda")
        fill_layer(layer, tables, old, latents=[x[:-1] for x in lat], keys=[k[:-1] for k in keys])
        pair.append(layer)
    new_lat = to_dev(np.stack([x[-1] for x in lat]))
    nk = np.stack([k[-1] for k in keys])
    new_key = to_dev(nk)
    return st, tables, lat, keys, pair, new_lat, new_key


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp4"])
def test_select_append_equals_append_then_select(dtype):
    """The append riding in the scan's launch: the cache rows it writes, the indices and the pool equal
    those of csa2_kv_append followed by csa2_index_select (the new key scored from the input gives the
    same score as from the cache), and the indices are exact against the oracle.  The lengths put the new
    position alone in a scan workgroup (2049), at a page start (4097), on the only position (1) and
    deep in a long row."""
    seq_lens = [70000, 2049, 1, 4097]
    B, K, P = len(seq_lens), 256, 256
    fp4 = dtype == "fp4"
    st, tables, lat, keys, (la, lb), new_lat, new_key = _append_case(dtype, seq_lens, 740)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    if fp4:
        q, w = to_dev(wl.q_idx_heads(st, 0, B)), to_dev(wl.w_idx(st, 0, B))
    else:
        q, w = to_dev(wl.q_idx(st, 0, B)), None
    idx_a, pool_a = csa2.csa2_index_select_append(la, batch, q, K, [(la, new_lat, None, new_key)], pool_blocks=P,
                                                  want_pool=True, w_idx=w)
    csa2.csa2_kv_append(lb, make_batch(tables, [n - 1 for n in seq_lens]), new_lat, None, new_key)
    idx_b, pool_b = csa2.csa2_index_select(lb, batch, q, K, csa2.FULL, pool_blocks=P, want_pool=True, w_idx=w)
    torch.cuda.synchronize()
    for name in ("codes", "scales", "idx_keys", "idx_scales"):
        ta, tb = getattr(la, name), getattr(lb, name)
        if ta is not None:
            assert torch.equal(ta, tb), name
    assert torch.equal(idx_a, idx_b) and torch.equal(pool_a, pool_b)
    got = idx_a.cpu().numpy()
    for b, n in enumerate(seq_lens):
        kf = (oracle.indexer.fp4_keys_to_f64(*oracle.fp4.fp4_pack(keys[b])) if fp4
              else oracle.indexer.keys_to_f64(keys[b], dtype))
        s = (oracle.indexer.index_scores(q.cpu().numpy()[b], kf, w.cpu().numpy()[b]) if fp4
             else oracle.indexer.index_scores(q.cpu().numpy()[b], kf))
        check_topk(got[b], dict(enumerate(s)), K, where=f"b={b}")


def test_select_append_serving_rows():
    """Mixed-serving style: the new token's key goes to a key-only pool and its latents to four layers' own
    pools, all in the scan's launch; every written row equals csa2_kv_append's, the indices equal the
    two-step path's."""
    st = wl.Streams(750)
    seq_lens = [9000, 300, 2048 * 3 + 1]
    B, K, L = len(seq_lens), 512, 4
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    old = [n - 1 for n in seq_lens]
    keys = [wl.idx_keys(st, b, n, "bf16") for b, n in enumerate(seq_lens)]
    lat = [[wl.latent_rows(st, l, b, n) for b, n in enumerate(seq_lens)] for l in range(L)]
    sides = []
    for _ in range(2):
        kp = csa2.PagedLayer(nb, idx_dtype="bf16", device="cuda")
        fill_layer(kp, tables, old, keys=[k[:-1] for k in keys])
        kv = []
        for l in range(L):
            x = csa2.PagedLayer(nb, device="cuda")
            fill_layer(x, tables, old, latents=[a[:-1] for a in lat[l]])
            kv.append(x)
        sides.append((kp, kv))
    new_key = to_dev(np.stack([k[-1] for k in keys]))
    new_lat = [to_dev(np.stack([a[-1] for a in lat[l]])) for l in range(L)]
    batch = make_batch(tables, seq_lens, max(seq_lens))
    q = to_dev(wl.q_idx(st, 0, B))
    kp, kv = sides[0]
    rows = [(kp, None, None, new_key)] + [(kv[l], new_lat[l], None, None) for l in range(L)]
    idx_a, _ = csa2.csa2_index_select_append(kp, batch, q, K, rows)
    kp2, kv2 = sides[1]
    prev = make_batch(tables, old)
    csa2.csa2_kv_append(kp2, prev, None, None, new_key)
    for l in range(L):
        csa2.csa2_kv_append(kv2[l], prev, new_lat[l])
    idx_b, _ = csa2.csa2_index_select(kp2, batch, q, K, csa2.FULL)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(kp.idx_keys, kp2.idx_keys)
    for l in range(L):
        assert torch.equal(kv[l].codes, kv2[l].codes) and torch.equal(kv[l].scales, kv2[l].scales), l
