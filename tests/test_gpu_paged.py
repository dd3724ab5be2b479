"""GPU parity of the paged append and the host page allocator in use."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import make_batch, to_dev

pytestmark = pytest.mark.gpu


def test_append_writes_packed_row_at_physical_slot():
    st = wl.Streams(70)
    seq_lens = [0, 63, 64, 200]
    pool = csa2.BlockPool(32)
    tables = np.full((4, 5), -1, dtype=np.int32)
    for b, n in enumerate(seq_lens):
        need = n // 64 + 1
        tables[b, :need] = pool.alloc(need)
    layer = csa2.PagedLayer(32, rope_dim=64, idx_dtype="bf16", device="cuda")
    lat = wl.latent_rows(st, 0, 0, 4)
    rope = wl.rope_rows(st, 0, 0, 4, 64)
    key = wl.idx_keys(st, 0, 4, "bf16")
    batch = make_batch(tables, seq_lens, 320)
    csa2.csa2_kv_append(layer, batch, to_dev(lat), to_dev(rope), to_dev(key))
    torch.cuda.synchronize()
    oc, os_ = oracle.fp4.fp4_pack(lat)
    codes, scales = layer.codes.cpu().numpy(), layer.scales.cpu().numpy()
    ropes, keys = layer.rope.cpu().numpy().view(np.uint16), layer.idx_keys.cpu().numpy().view(np.uint16)
    written = set()
    for b, p in enumerate(seq_lens):
        r = oracle.paged.physical_row(tables, b, p)
        written.add(r)
        assert np.array_equal(codes[r], oc[b]) and np.array_equal(scales[r], os_[b])
        assert np.array_equal(ropes[r], rope[b]) and np.array_equal(keys[r], key[b])
    others = [r for r in range(32 * 64) if r not in written]
    assert not codes[others].any() and not scales[others].any()


def test_append_skips_unmapped_pages():
    layer = csa2.PagedLayer(2, device="cuda")
    tables = np.array([[0, -1], [1, 5]], dtype=np.int32)  # page 1 of seq 0 unmapped; id 5 out of pool
    batch = make_batch(tables, [64, 64], 128)
    lat = np.ones((2, 512), dtype=np.float32)
    csa2.csa2_kv_append(layer, batch, to_dev(lat))
    torch.cuda.synchronize()
    assert not layer.codes.cpu().numpy().any()
