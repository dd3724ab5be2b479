"""The allocation-free attention entry point (csa2_sparse_fp4_decode_attn_layers_noalloc) called through the
C ABI: two calls in a row, the second on a smaller problem, each equal to the workspace entry point's result
on the same arguments (the same kernels and split choice, so the same bits) and within the attention bar of
the oracle; a problem whose usual split count would overflow the scratch runs with fewer splits."""

import ctypes
import math

import numpy as np
import pytest
import torch

from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import ATTN_TOL, build_tables, fill_layer, make_batch, oracle_attention_rows, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, seq_lens, L, H, K):
    st = wl.Streams(seed)
    B = len(seq_lens)
    tables, nb = build_tables(st, seq_lens, True)
    lat = [[wl.latent_rows(st, l, b, n) for b, n in enumerate(seq_lens)] for l in range(L)]
    layers = []
    for l in range(L):
        layer = csa2.PagedLayer(nb, device="cuda")
        fill_layer(layer, tables, seq_lens, latents=lat[l])
        layers.append(layer)
    rng = np.random.default_rng(seed)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b, n in enumerate(seq_lens):
        m = min(n, K)
        idx[b, :m] = rng.choice(n, size=m, replace=False)
    q = [wl.q_heads(st, l, B, H, 512) for l in range(L)]
    return make_batch(tables, seq_lens, max(seq_lens)), layers, lat, to_dev(idx), idx, q


def _noalloc(batch, layers, q_d, idx_d, sigma, H, K):
    B = batch.batch
    outs = [torch.full((B, H, 512), float("nan"), dtype=torch.float32, device="cuda") for _ in layers]
    lses = [torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda") for _ in layers]
    kvs = [x.struct() for x in layers]
    arr = (csa2.AttnLayerC * len(layers))(*[
        csa2.AttnLayerC(ctypes.pointer(kv), csa2._ptr(q), csa2._ptr(idx_d), csa2._ptr(o), csa2._ptr(ls), None, None)
        for kv, q, o, ls in zip(kvs, q_d, outs, lses)])
    sq = batch.struct()
    st = csa2.lib().csa2_sparse_fp4_decode_attn_layers_noalloc(arr, len(layers), ctypes.byref(sq), H, K, sigma,
                                                               csa2._stream())
    assert st == csa2.OK, st
    return outs, lses


def test_noalloc_matches_workspace_entry_point_twice():
    sigma = 1 / math.sqrt(512)
    # first call: the 1M-step shape at a smaller length (4 layers, batch 1, 64 heads, K 2048: 16 splits);
    # second call: a smaller problem (2 layers, batch 3, 16 heads, K 256), which reuses the same scratch
    for seed, seq_lens, L, H, K in ((900, [30000], 4, 64, 2048), (901, [700, 5000, 64], 2, 16, 256)):
        batch, layers, lat, idx_d, idx, q = _case(seed, seq_lens, L, H, K)
        q_d = [to_dev(x) for x in q]
        outs, lses = _noalloc(batch, layers, q_d, idx_d, sigma, H, K)
        ref_o, ref_l = csa2.csa2_sparse_fp4_decode_attn_layers([(layers[l], q_d[l], idx_d) for l in range(L)], batch,
                                                               sigma)
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(outs[l], ref_o[l]) and torch.equal(lses[l], ref_l[l]), (seed, l)
            for b, n in enumerate(seq_lens):
                o_out, _ = oracle_attention_rows(lat[l][b], None, q[l][b], idx[b], n, sigma)
                assert float(np.max(np.abs(outs[l].cpu().numpy()[b] - o_out))) <= ATTN_TOL, (seed, l, b)


def test_noalloc_lowers_splits_to_fit_its_scratch():
    """Batch 16 x 64 heads at K 2048: the workspace entry point's 16 splits need more than the 32 MiB scratch
    (16 x 64 x 16 partial rows of 2 KB, plus their m and l), so the allocation-free call runs with fewer; same
    result within the rounding of a different split (each within ~2e-5 of the exact one) and within the
    attention bar of the oracle."""
    sigma = 1 / math.sqrt(512)
    seq_lens, L, H, K = [2500 + 97 * b for b in range(16)], 1, 64, 2048
    n = ctypes.c_size_t()
    assert csa2.lib().csa2_attn_layers_workspace_size(L, len(seq_lens), H, K, 512, 0, ctypes.byref(n)) == csa2.OK
    assert n.value > 32 << 20
    batch, layers, lat, idx_d, idx, q = _case(902, seq_lens, L, H, K)
    q_d = [to_dev(x) for x in q]
    outs, lses = _noalloc(batch, layers, q_d, idx_d, sigma, H, K)
    ref_o, ref_l = csa2.csa2_sparse_fp4_decode_attn_layers([(layers[0], q_d[0], idx_d)], batch, sigma)
    torch.cuda.synchronize()
    assert bool(((outs[0] - ref_o[0]).abs() <= 5e-5 * ref_o[0].abs().clamp(min=1.0)).all())
    assert float((lses[0] - ref_l[0]).abs().max()) <= 1e-5
    for b, n_b in enumerate(seq_lens):
        o_out, _ = oracle_attention_rows(lat[0][b], None, q[0][b], idx[b], n_b, sigma)
        assert float(np.max(np.abs(outs[0].cpu().numpy()[b] - o_out))) <= ATTN_TOL, b


def test_noalloc_rejects_beyond_its_scratch():
    """A problem whose partials exceed the 32 MiB scratch is refused before any launch."""
    n = ctypes.c_size_t()
    assert csa2.lib().csa2_attn_layers_workspace_size(20, 64, 128, 4096, 512, 1, ctypes.byref(n)) == csa2.OK
    assert n.value > 32 << 20
    kv = csa2.KvLayer(codes=256, scales=256, rope=None, idx_keys=None, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    w = csa2.SwaWindow(codes=256, scales=256, batch=64)
    arr = (csa2.AttnLayerC * 20)(*[csa2.AttnLayerC(ctypes.pointer(kv), 256, 256, 256, None, ctypes.pointer(w), None)
                                   for _ in range(20)])
    sq = csa2.Seqs(block_table=256, max_blocks_per_seq=1, seq_lens=256, batch=64, max_seq_len=64)
    assert csa2.lib().csa2_sparse_fp4_decode_attn_layers_noalloc(arr, 20, ctypes.byref(sq), 128, 4096, 0.1,
                                                                 None) == csa2.ERR_WORKSPACE
