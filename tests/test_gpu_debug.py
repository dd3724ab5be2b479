"""Debug checks (device-side checks of the documented input contracts): every flag is raised by an input that
breaks its contract and by nothing else; with the checks off nothing is recorded.  Every input here is one the
kernels handle without faulting (skipped entries stay skipped, out-of-range values give NaN results)."""

import math

import numpy as np
import pytest
import torch

from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import build_tables, fill_layer, make_batch, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture()
def checks():
    csa2.csa2_debug_checks(True)
    csa2.csa2_debug_flags()  # start clean
    yield
    csa2.csa2_debug_flags()
    csa2.csa2_debug_checks(False)


def _attn_case(seed=950):
    st = wl.Streams(seed)
    seq_lens = [3000, 700]
    tables, nb = build_tables(st, seq_lens, True)
    layer = csa2.PagedLayer(nb, rope_dim=64, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=[wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)],
               ropes=[wl.rope_rows(st, 0, b, n, 64) for b, n in enumerate(seq_lens)])
    q = wl.q_heads(st, 0, 2, 64, 576)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(n, 256, replace=False) for n in seq_lens]).astype(np.int32)
    idx[:, :8] = -1  # padding is legal
    return st, tables, seq_lens, layer, q, idx


def test_clean_inputs_raise_nothing(checks):
    st, tables, seq_lens, layer, q, idx = _attn_case()
    batch = make_batch(tables, seq_lens, max(seq_lens))
    csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q), to_dev(idx), 1 / math.sqrt(576))
    keys = csa2.PagedLayer(layer.num_blocks, idx_dtype="bf16", device="cuda")
    fill_layer(keys, tables, seq_lens, keys=[wl.idx_keys(st, b, n, "bf16") for b, n in enumerate(seq_lens)])
    csa2.csa2_index_select(keys, batch, to_dev(wl.q_idx(st, 0, 2)), 64, csa2.FULL)
    csa2.csa2_fp4_pack(to_dev(wl.latent_rows(st, 0, 0, 100)))
    assert csa2.csa2_debug_flags() == 0


def test_each_flag(checks):
    st, tables, seq_lens, layer, q, idx = _attn_case()
    sigma = 1 / math.sqrt(576)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    # a query value beyond fp16's range
    qb = q.copy()
    qb[1, 5, 100] = wl.to_bf16_bits(np.array([1.0e5], dtype=np.float32))[0]
    csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(qb), to_dev(idx), sigma)
    assert csa2.csa2_debug_flags() == csa2.DBG_Q_RANGE
    # selected indices past the length and below -1
    ib = idx.copy()
    ib[0, 10], ib[1, 11] = seq_lens[0], -7
    csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q), to_dev(ib), sigma)
    assert csa2.csa2_debug_flags() == csa2.DBG_INDEX
    # a visible page mapped outside the pool
    tb = tables.copy()
    tb[0, 3] = layer.num_blocks + 5
    csa2.csa2_sparse_fp4_decode_attn(layer, make_batch(tb, seq_lens, max(seq_lens)), to_dev(q),
                                     to_dev(np.full_like(idx, 200)), sigma)
    assert csa2.csa2_debug_flags() == csa2.DBG_PAGE
    # a length beyond max_seq_len
    csa2.csa2_sparse_fp4_decode_attn(layer, make_batch(tables, [seq_lens[0], seq_lens[0]], seq_lens[0] - 1),
                                     to_dev(q), to_dev(idx), sigma)
    assert csa2.csa2_debug_flags() & csa2.DBG_SEQ_LEN
    # non-finite values into the pack and the append
    x = wl.latent_rows(st, 0, 0, 40)
    x[7, 3] = np.nan
    csa2.csa2_fp4_pack(to_dev(x))
    assert csa2.csa2_debug_flags() == csa2.DBG_NONFINITE
    lat = np.zeros((2, 512), np.float32)
    lat[1, 0] = np.inf
    csa2.csa2_kv_append(layer, make_batch(tables, [10, 10]), to_dev(lat), to_dev(np.zeros((2, 64), np.uint16)))
    assert csa2.csa2_debug_flags() == csa2.DBG_NONFINITE
    # a non-finite score given to the top-K
    sc = np.random.default_rng(1).standard_normal((2, 5000)).astype(np.float32)
    sc[1, 17] = np.inf
    csa2.csa2_topk(to_dev(sc), to_dev(np.array([5000, 5000], np.int32)), 64)
    assert csa2.csa2_debug_flags() == csa2.DBG_SCORE


def test_checks_off_record_nothing():
    csa2.csa2_debug_checks(False)
    st, tables, seq_lens, layer, q, idx = _attn_case()
    qb = q.copy()
    qb[0, 0, 0] = wl.to_bf16_bits(np.array([1.0e5], dtype=np.float32))[0]
    csa2.csa2_sparse_fp4_decode_attn(layer, make_batch(tables, seq_lens, max(seq_lens)), to_dev(qb), to_dev(idx),
                                     0.05)
    torch.cuda.synchronize()
    assert csa2.csa2_debug_flags() == 0
