"""The decoder's CSA2 schedule end to end on one KV source (P1 CSA2 layer layout: decoder layers in
groups of 4, the first group Full + 3 Reuse, later groups Reindex + 3 Reuse; top-K 512; 32 x 128
FP4 indexer): append, selection with the 2048 x 8 pool, Reindex, Reuse and attention, each checked
against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import ATTN_TOL, LSE_TOL, build_tables, check_topk, fill_layer, make_batch, oracle_attention_rows, to_dev

pytestmark = pytest.mark.gpu


def test_decoder_schedule_two_groups():
    st = wl.Streams(60)
    seq_lens = [30000, 5000, 513]
    B, K, P, G, L, H = len(seq_lens), 512, 2048, 4, 8, 64
    sigma = 1 / math.sqrt(512)
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    lat = [wl.latent_rows(st, 0, b, n + 1) for b, n in enumerate(seq_lens)]   # the last row is appended
    keys = [wl.idx4_keys(st, b, n + 1) for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, idx_dtype="fp4", device="cuda")
    fill_layer(layer, tables, seq_lens, latents=[x[:-1] for x in lat], keys=[k[:-1] for k in keys])
    # append the new token at position n, then every layer sees n + 1 positions
    csa2.csa2_kv_append(layer, make_batch(tables, seq_lens), to_dev(np.stack([x[-1] for x in lat])), None,
                        to_dev(np.stack([k[-1] for k in keys])))
    n1 = [n + 1 for n in seq_lens]
    batch = make_batch(tables, n1, max(n1))
    qi = [wl.q_idx_heads(st, l, B) for l in range(L)]
    wi = [wl.w_idx(st, l, B) for l in range(L)]
    q = [wl.q_heads(st, l, B, H, 512) for l in range(L)]
    sel, pool, outs = {}, None, {}
    for l0 in range(0, L, G):
        if l0 == 0:
            idx, pool = csa2.csa2_index_select(layer, batch, to_dev(qi[l0]), K, csa2.FULL, pool_blocks=P,
                                               want_pool=True, w_idx=to_dev(wi[l0]))
        else:
            idx, _ = csa2.csa2_index_select(layer, batch, to_dev(qi[l0]), K, csa2.REINDEX, pool_in=pool,
                                            pool_blocks=P, w_idx=to_dev(wi[l0]))
        sel[l0] = idx
        for l in range(l0, l0 + G):  # the lead layer and its Reuse layers attend over the same indices
            outs[l] = csa2.csa2_sparse_fp4_decode_attn(layer, batch, to_dev(q[l]), idx, sigma)
    torch.cuda.synchronize()
    pool = pool.cpu().numpy()
    for b, n in enumerate(n1):
        kf = oracle.indexer.fp4_keys_to_f64(*oracle.fp4.fp4_pack(keys[b]))
        s0 = oracle.indexer.index_scores(qi[0][b], kf, wi[0][b])
        check_topk(pool[b], dict(enumerate(oracle.indexer.block_scores_fast(s0))), P, where=f"pool b={b}")
        for l0, idx in sel.items():
            idx = idx.cpu().numpy()[b]
            if l0 == 0:
                check_topk(idx, dict(enumerate(s0)), K, where=f"full b={b}")
            else:  # Reindex over the GPU's pool (checked above)
                pos = oracle.indexer.pool_positions(pool[b][pool[b] >= 0], n)
                s = oracle.indexer.index_scores(qi[l0][b], kf[pos], wi[l0][b])
                check_topk(idx, dict(zip(pos.tolist(), s)), K, where=f"reindex l={l0} b={b}")
            # attention of the lead and its Reuse layers over the selected entries
            for l in range(l0, l0 + G):
                o_out, o_lse = oracle_attention_rows(lat[b], None, q[l][b], oracle.indexer.reuse_select(idx), n,
                                                     sigma)
                out, lse = outs[l][0].cpu().numpy()[b], outs[l][1].cpu().numpy()[b]
                assert float(np.max(np.abs(out - o_out))) <= ATTN_TOL, (l, b)
                assert float(np.max(np.abs(lse - o_lse))) <= LSE_TOL, (l, b)
