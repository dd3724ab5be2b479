"""Canary guards and run-twice determinism: every output buffer of the hot path is carved out of a larger
allocation whose margins hold a fixed byte pattern; after the calls the margins must be unchanged (no write
lands outside its output), and a second identical call must reproduce every output bit for bit."""

import math

import numpy as np
import pytest
import torch

from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import build_tables, fill_layer, make_batch, to_dev

pytestmark = pytest.mark.gpu

MARGIN = 4096  # bytes of canary on each side
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape`/`dtype` inside a byte buffer with MARGIN canary bytes on both sides."""

    def __init__(self, shape, dtype, device="cuda"):
        itemsize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * itemsize
        self.raw = torch.full((2 * MARGIN + n,), PATTERN, dtype=torch.uint8, device=device)
        self.t = self.raw[MARGIN:MARGIN + n].view(dtype).view(shape)
        self.n = n

    def intact(self):
        head, tail = self.raw[:MARGIN], self.raw[MARGIN + self.n:]
        return bool((head == PATTERN).all()) and bool((tail == PATTERN).all())


def _setup(seed=960):
    st = wl.Streams(seed)
    seq_lens = [40000, 700, 2049]
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    layer = csa2.PagedLayer(nb, idx_dtype="bf16", device="cuda")
    fill_layer(layer, tables, seq_lens, latents=[wl.latent_rows(st, 0, b, n) for b, n in enumerate(seq_lens)],
               keys=[wl.idx_keys(st, b, n, "bf16") for b, n in enumerate(seq_lens)])
    return st, seq_lens, tables, layer


def test_outputs_stay_inside_their_buffers_and_repeat_exactly():
    st, seq_lens, tables, layer = _setup()
    B, K, P, H = len(seq_lens), 512, 256, 64
    batch = make_batch(tables, seq_lens, max(seq_lens))
    qi = [to_dev(wl.q_idx(st, l, B)) for l in range(3)]
    q = [to_dev(wl.q_heads(st, l, B, H, 512)) for l in range(3)]
    sigma = 1 / math.sqrt(512)

    def run():
        g = {name: Guarded(shape, dt) for name, shape, dt in (
            ("idx0", (B, K), torch.int32), ("pool", (B, P), torch.int32), ("idx1", (B, K), torch.int32),
            ("idx2", (B, K), torch.int32), ("out0", (B, H, 512), torch.float32), ("out1", (B, H, 512), torch.float32),
            ("out2", (B, H, 512), torch.float32), ("lse0", (B, H), torch.float32), ("lse1", (B, H), torch.float32),
            ("lse2", (B, H), torch.float32), ("codes", (100, 256), torch.uint8), ("scales", (100, 32), torch.uint8),
            ("topk", (B, 64), torch.int32))}
        csa2.csa2_index_select(layer, batch, qi[0], K, csa2.FULL, pool_blocks=P, want_pool=True,
                               indices=g["idx0"].t, pool_out=g["pool"].t)
        csa2.csa2_index_reindex_layers(layer, batch, [(qi[1], None), (qi[2], None)], K, g["pool"].t, P,
                                       indices=[g["idx1"].t, g["idx2"].t])
        csa2.csa2_sparse_fp4_decode_attn_layers(
            [(layer, q[0], g["idx0"].t), (layer, q[1], g["idx1"].t), (layer, q[2], g["idx2"].t)], batch, sigma,
            outs=[g["out0"].t, g["out1"].t, g["out2"].t], lses=[g["lse0"].t, g["lse1"].t, g["lse2"].t])
        csa2.csa2_fp4_pack_into(to_dev(wl.latent_rows(st, 5, 0, 100)), g["codes"].t, g["scales"].t)
        sc = to_dev(np.random.default_rng(3).standard_normal((B, 3000)).astype(np.float32))
        ws = csa2.workspace(csa2.topk_workspace_bytes(B, 3000, 64))
        res = csa2.lib().csa2_topk(csa2._ptr(sc), 3000, csa2._ptr(to_dev(np.array([3000, 10, 2999], np.int32))), B,
                                   3000, 64, csa2._ptr(g["topk"].t), csa2._ptr(ws), ws.numel(), csa2._stream())
        assert res == csa2.OK
        torch.cuda.synchronize()
        return g

    first = run()
    for name, x in first.items():
        assert x.intact(), f"{name}: a write landed outside the output"
    second = run()
    for name in first:
        assert torch.equal(first[name].t, second[name].t), f"{name}: a second identical call differs"
