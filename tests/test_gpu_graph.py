"""A decode step captured as a HIP graph gives, on every replay, the bytes the same step gives when
launched eagerly (the benchmark replays captured steps).  Between replays the program runs eager work of
its own and synchronizes."""

import math

import numpy as np
import pytest
import torch

from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import build_tables, fill_layer, make_batch, to_dev

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    st = wl.Streams(110)
    seq_lens = [20000, 3001]
    B, H, K, P = len(seq_lens), 64, 512, 2048
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)]
    keys = [wl.idx_keys(st, b, n, "bf16") for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, idx_dtype="bf16", device="cuda")
    fill_layer(layer, tables, seq_lens, latents=lat, keys=keys)
    n1 = [n + 1 for n in seq_lens]
    batch_prev, batch = make_batch(tables, seq_lens), make_batch(tables, n1, max(n1))
    new_lat = to_dev(wl.latent_rows(st, 0, 9, B))
    new_key = to_dev(wl.idx_keys(st, 9, B, "bf16"))
    q_idx = [to_dev(wl.q_idx(st, l, B)) for l in range(2)]
    q = [to_dev(wl.q_heads(st, l, B, H, 512)) for l in range(2)]
    sel_ws = csa2.workspace(csa2.index_select_workspace_bytes(B, max(n1), K, P))
    attn_ws = csa2.workspace(csa2.attn_workspace_bytes(B, H, K))
    idx = torch.empty((2, B, K), dtype=torch.int32, device="cuda")
    pool = torch.empty((B, P), dtype=torch.int32, device="cuda")
    out = torch.empty((2, B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((2, B, H), dtype=torch.float32, device="cuda")
    sigma = 1 / math.sqrt(512)

    def step():
        csa2.csa2_kv_append(layer, batch_prev, new_lat, idx_key=new_key)
        csa2.csa2_index_select(layer, batch, q_idx[0], K, csa2.FULL, pool_blocks=P, want_pool=True, ws=sel_ws,
                               indices=idx[0], pool_out=pool)
        csa2.csa2_index_select(layer, batch, q_idx[1], K, csa2.REINDEX, pool_in=pool, pool_blocks=P, ws=sel_ws,
                               indices=idx[1])
        for l in range(2):
            csa2.csa2_sparse_fp4_decode_attn(layer, batch, q[l], idx[l], sigma, ws=attn_ws, out=out[l], lse=lse[l])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, pool, out, lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (idx, pool, out, lse):
            t.fill_(-7)  # eager work between replays; any stale output would show
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip((idx, pool, out, lse), ref):
            assert torch.equal(a, r), f"replay {rep}"


def test_captured_window_attention_replays_match_eager():
    """The attention call that takes the sliding window as extra splits and appends the current token's window
    entry (a ring write inside the kernel) replays from a graph with the eager bytes, ring included."""
    st = wl.Streams(111)
    seq_lens = [20000, 3001]
    B, H, K = len(seq_lens), 64, 2048
    tables, nb = build_tables(st, seq_lens, True)
    lat = [wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)]
    layer = csa2.PagedLayer(nb, device="cuda")
    fill_layer(layer, tables, seq_lens, latents=lat)
    batch = make_batch(tables, seq_lens, max(seq_lens))
    rng = np.random.default_rng(5)
    idx = to_dev(np.stack([rng.choice(n, size=K, replace=False).astype(np.int32) for n in seq_lens]))
    q = to_dev(wl.q_heads(st, 0, B, H, 512))
    ring = csa2.SwaRing(B)
    for j in range(127):  # positions n - 128 .. n - 2; the call appends n - 1
        pos = to_dev(np.array([n - 128 + j for n in seq_lens], dtype=np.int32))
        csa2.csa2_swa_append(ring, pos, to_dev(wl.latent_rows(st, 1, j, B)))
    new = to_dev(wl.latent_rows(st, 1, 127, B))
    ws = csa2.workspace(csa2.attn_swa_workspace_bytes(B, H, K))
    out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    sigma = 1 / math.sqrt(512)

    def step():
        csa2.csa2_sparse_fp4_decode_attn_swa(layer, batch, q, idx, sigma, ring, new_latent=new, ws=ws, out=out,
                                             lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, ring.codes, ring.scales)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    slots = [(n - 1) % 128 for n in seq_lens]
    for rep in range(3):
        out.fill_(-7)
        lse.fill_(-7)
        for b, sl in enumerate(slots):  # the appended slot is written again by every replay
            ring.codes[b, sl].fill_(0)
            ring.scales[b, sl] = -1.0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip((out, lse, ring.codes, ring.scales), ref):
            assert torch.equal(a, r), f"replay {rep}"
