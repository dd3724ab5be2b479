"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and its host-side validation and page allocator behave as
documented (no GPU work is launched by any call here)."""

import ctypes
import glob
import os
import re

import pytest

from sparse_attention_fp4_kv_amd import csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    """These checks need the built library: build it when it is missing (hipcc cross-compiles without a GPU),
    and fail, not skip, when that is impossible."""
    if not os.path.exists(csa2.LIB_PATH):
        from sparse_attention_fp4_kv_amd import build_lib

        build_lib.build()
    assert os.path.exists(csa2.LIB_PATH), "libcsa2.so could not be built"


def needs_lib(f):
    return f


def header_functions():
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_header_lists_the_entry_points():
    names = header_functions()
    for must in ("csa2_fp4_pack", "csa2_fp4_unpack", "csa2_kv_append", "csa2_ced_kv_project", "csa2_index_select",
                 "csa2_topk", "csa2_sparse_fp4_decode_attn", "csa2_block_pool_create"):
        assert must in names
    assert set(names) == set(csa2.SIGNATURES)


@needs_lib
def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(csa2.LIB_PATH)
    for name in header_functions():
        assert hasattr(raw, name), name
    assert csa2.lib().csa2_abi_version() == 6
    assert csa2.lib().csa2_status_string(3) == b"workspace missing or too small"


@needs_lib
def test_validation_rejects_before_launch():
    L = csa2.lib()
    s = None
    assert L.csa2_fp4_pack(None, 4, 15, None, None, s) == csa2.ERR_INVALID_ARG
    assert L.csa2_fp4_pack(None, -1, 16, None, None, s) == csa2.ERR_INVALID_ARG
    assert L.csa2_fp4_pack(None, 0, 16, None, None, s) == csa2.OK  # empty is a no-op
    assert L.csa2_fp4_pack(None, 4, 16, None, None, s) == csa2.ERR_INVALID_ARG
    assert L.csa2_ced_kv_project(None, 4, 100, 1, None, None, None, None, None, None, s) == csa2.ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert L.csa2_topk_workspace_size(1, 100, 0, ctypes.byref(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_topk_workspace_size(1, 100, 4097, ctypes.byref(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_topk_workspace_size(2, 1000, 64, ctypes.byref(n)) == csa2.OK and n.value > 0
    assert L.csa2_attn_workspace_size(1, 20, 64, 512, ctypes.byref(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_attn_workspace_size(1, 64, 2048, 512, ctypes.byref(n)) == csa2.OK
    # a layer with the wrong page size is rejected
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=16, num_blocks=1, block_tokens=32, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    sq = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=1, max_seq_len=64)
    assert L.csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), 16, None, 16, s) == csa2.ERR_INVALID_ARG
    kv.block_tokens = 64
    sq.max_seq_len = 65  # beyond max_blocks_per_seq * 64
    assert L.csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), 16, None, 16, s) == csa2.ERR_INVALID_ARG
    sq.max_seq_len = 64
    # too-small workspace
    assert L.csa2_index_select(ctypes.byref(kv), ctypes.byref(sq), 16, None, 8, csa2.FULL, None, None, 0, 0, 16, 256, 1,
                               s) == csa2.ERR_WORKSPACE
    # Reindex without a pool
    assert L.csa2_index_select(ctypes.byref(kv), ctypes.byref(sq), 16, None, 8, csa2.REINDEX, None, None, 16, 8, 16, 256,
                               1 << 30, s) == csa2.ERR_INVALID_ARG
    # weights are for FP4 keys only
    assert L.csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), 16, 16, 16, s) == csa2.ERR_INVALID_ARG
    # FP4 keys: 128 dims, 1..32 heads, scales present, weights required
    kv.idx_dtype, kv.idx_dim, kv.idx_heads, kv.idx_scales = csa2.FP4, 128, 32, 16
    assert L.csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), 16, None, 16, s) == csa2.ERR_INVALID_ARG
    for field, bad in (("idx_dim", 64), ("idx_heads", 33), ("idx_heads", 0), ("idx_scales", None)):
        good = getattr(kv, field)
        setattr(kv, field, bad)
        assert L.csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), 16, 16, 16, s) == csa2.ERR_INVALID_ARG
        setattr(kv, field, good)
    assert L.csa2_index_select(ctypes.byref(kv), ctypes.byref(sq), 16, 16, 8, csa2.FULL, None, None, 0, 0, 16, 256, 1,
                               s) == csa2.ERR_WORKSPACE


@needs_lib
def test_finish_validation_rejects_before_launch():
    L = csa2.lib()
    s = None
    fin = csa2.KvFinish(gamma=16, eps=1e-6, rope_theta=10000.0, w_idx=16)
    P = ctypes.byref
    # tokens == 0 is a no-op once the arguments are valid
    assert L.csa2_kv_finish_rows(None, 0, 1, 0, P(fin), 16, 16, 16, 16, None, None, s) == csa2.OK
    # positions beyond 2^24
    assert L.csa2_kv_finish_rows(16, 10, 1, (1 << 24) - 5, P(fin), 16, 16, 16, 16, None, None,
                                 s) == csa2.ERR_INVALID_ARG
    # the key outputs are required with W_idx and refused without it
    assert L.csa2_kv_finish_rows(16, 10, 1, 0, P(fin), 16, 16, None, 16, None, None, s) == csa2.ERR_INVALID_ARG
    fin.w_idx = None
    assert L.csa2_kv_finish_rows(16, 10, 1, 0, P(fin), 16, 16, 16, 16, None, None, s) == csa2.ERR_INVALID_ARG
    for field, bad in (("eps", 0.0), ("eps", -1.0), ("rope_theta", -1.0), ("gamma", None), ("gamma", 8)):
        good = getattr(fin, field)
        setattr(fin, field, bad)
        assert L.csa2_kv_finish_rows(16, 10, 1, 0, P(fin), 16, 16, None, None, None, None,
                                     s) == csa2.ERR_INVALID_ARG, field
        setattr(fin, field, good)
    assert L.csa2_kv_finish_rows(16, 10, 1, 0, None, 16, 16, None, None, None, None, s) == csa2.ERR_INVALID_ARG
    # CED with the finish needs the hand-over buffer
    assert L.csa2_ced_kv_project_finished(16, 10, 64, 1, 16, P(fin), 0, None, 16, 16, None, None,
                                          s) == csa2.ERR_INVALID_ARG
    # the finishing append: a layer with bf16 keys cannot take a key projected from the main KV
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=16, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    sq = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=1, max_seq_len=64)
    assert L.csa2_kv_append_finished(P(kv), P(sq), 16, P(fin), s) == csa2.ERR_INVALID_ARG
    # FP4 keys need W_idx
    kv.idx_dtype, kv.idx_dim, kv.idx_heads, kv.idx_scales = csa2.FP4, 128, 32, 16
    assert L.csa2_kv_append_finished(P(kv), P(sq), 16, P(fin), s) == csa2.ERR_INVALID_ARG


@needs_lib
def test_swa_validation_rejects_before_launch():
    L = csa2.lib()
    P = ctypes.byref
    w = csa2.SwaWindow(codes=16, scales=16, batch=2)
    assert L.csa2_swa_append(P(w), 16, 3, 16, None) == csa2.ERR_INVALID_ARG  # beyond the ring's batch
    assert L.csa2_swa_append(P(w), 16, 0, None, None) == csa2.OK
    for heads, qd in ((8, 512), (24, 512), (144, 512), (16, 520)):
        assert L.csa2_swa_attn_merge(P(w), 16, 1, 16, heads, qd, 0.1, 16, 16, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_swa_attn_merge(P(w), 16, 1, 16, 16, 512, 0.0, 16, 16, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_swa_attn_merge(P(w), 16, 1, 16, 16, 512, 0.1, 16, None, None) == csa2.ERR_INVALID_ARG


@needs_lib
def test_attn_swa_validation_rejects_before_launch():
    L = csa2.lib()
    P = ctypes.byref
    n, m = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.csa2_attn_swa_workspace_size(1, 20, 64, 512, P(n)) == csa2.ERR_INVALID_ARG
    # the window adds four partials per head: batch 1 needs more workspace than the plain attention
    assert L.csa2_attn_swa_workspace_size(1, 64, 2048, 512, P(n)) == csa2.OK
    assert L.csa2_attn_workspace_size(1, 64, 2048, 512, P(m)) == csa2.OK and n.value > m.value
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=16, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    sq = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=2, max_seq_len=64)
    f = L.csa2_sparse_fp4_decode_attn_swa
    w = csa2.SwaWindow(codes=16, scales=16, batch=2)
    small = csa2.SwaWindow(codes=16, scales=16, batch=1)
    nocodes = csa2.SwaWindow(codes=None, scales=16, batch=2)
    assert f(P(kv), P(sq), 16, 64, 16, 64, 0.1, None, None, 16, None, 256, 64, None) == csa2.ERR_INVALID_ARG
    assert f(P(kv), P(sq), 16, 64, 16, 64, 0.1, P(small), None, 16, None, 256, 64, None) == csa2.ERR_INVALID_ARG
    assert f(P(kv), P(sq), 16, 64, 16, 64, 0.1, P(nocodes), None, 16, None, 256, 64, None) == csa2.ERR_INVALID_ARG
    assert f(P(kv), P(sq), 16, 24, 16, 64, 0.1, P(w), None, 16, None, 256, 64, None) == csa2.ERR_INVALID_ARG
    assert f(P(kv), P(sq), 16, 64, 16, 64, 0.1, P(w), None, 16, None, 256, 64, None) == csa2.ERR_WORKSPACE
    # a misaligned appended entry
    assert f(P(kv), P(sq), 16, 64, 16, 64, 0.1, P(w), 4, 16, None, 256, 1 << 20, None) == csa2.ERR_INVALID_ARG


@needs_lib
def test_block_pool():
    p = csa2.BlockPool(5)
    a = p.alloc(3)
    assert a == [0, 1, 2] and p.num_free == 2
    with pytest.raises(csa2.Csa2Error):
        p.alloc(3)  # not enough: nothing taken
    assert p.num_free == 2
    with pytest.raises(csa2.Csa2Error):
        p.free([1, 1])  # duplicate
    with pytest.raises(csa2.Csa2Error):
        p.free([4])  # already free
    assert p.num_free == 2
    p.free([1])
    assert p.num_free == 3 and p.alloc(1) == [1]
    p.close()


@needs_lib
def test_multi_layer_validation_rejects_before_launch():
    L = csa2.lib()
    P = ctypes.byref
    n = ctypes.c_size_t()
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=16, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    sq = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=1, max_seq_len=64)
    # attention over layers: 1..20 layers, one rope width, windows on all layers or none
    assert L.csa2_attn_layers_workspace_size(0, 1, 64, 2048, 512, 0, P(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_attn_layers_workspace_size(21, 1, 64, 2048, 512, 0, P(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_attn_layers_workspace_size(4, 1, 64, 2048, 512, 0, P(n)) == csa2.OK
    four = n.value
    assert L.csa2_attn_layers_workspace_size(1, 1, 64, 2048, 512, 0, P(n)) == csa2.OK and n.value <= four
    rope = csa2.KvLayer(codes=16, scales=16, rope=16, idx_keys=None, num_blocks=1, block_tokens=64, latent_dim=512,
                        rope_dim=64, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    w = csa2.SwaWindow(codes=16, scales=16, batch=1)
    mk = lambda layer, win=None, nl=None: csa2.AttnLayerC(ctypes.pointer(layer), 16, 16, 16, None,
                                                           ctypes.pointer(win) if win else None, nl)
    f = L.csa2_sparse_fp4_decode_attn_layers
    arr = (csa2.AttnLayerC * 2)(mk(kv), mk(rope))
    assert f(arr, 2, P(sq), 64, 64, 0.1, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG  # mixed rope widths
    arr = (csa2.AttnLayerC * 2)(mk(kv), mk(kv, w))
    assert f(arr, 2, P(sq), 64, 64, 0.1, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG  # window on one layer only
    arr = (csa2.AttnLayerC * 1)(mk(kv, None, 16))
    assert f(arr, 1, P(sq), 64, 64, 0.1, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG  # new entry without a window
    arr = (csa2.AttnLayerC * 2)(mk(kv), mk(kv))
    assert f(arr, 0, P(sq), 64, 64, 0.1, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    assert f(arr, 2, P(sq), 24, 64, 0.1, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    assert f(arr, 2, P(sq), 64, 64, 0.1, 256, 1, None) == csa2.ERR_WORKSPACE
    # Reindex over layers: 1..8 layers, a pool, the keys' query kind
    assert L.csa2_index_reindex_layers_workspace_size(9, 1, 64, 2048, 8, P(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_reindex_layers_workspace_size(3, 1, 64, 2048, 4, P(n)) == csa2.ERR_INVALID_ARG
    assert L.csa2_index_reindex_layers_workspace_size(3, 1, 64, 2048, 8, P(n)) == csa2.OK
    three = n.value
    assert L.csa2_index_reindex_layers_workspace_size(1, 1, 64, 2048, 8, P(n)) == csa2.OK and 3 * n.value == three
    g = L.csa2_index_reindex_layers
    qs = (csa2.ReindexQueryC * 2)(csa2.ReindexQueryC(16, None, 16), csa2.ReindexQueryC(16, None, 16))
    assert g(P(kv), P(sq), qs, 2, 64, None, 2048, 8, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG  # no pool
    assert g(P(kv), P(sq), qs, 2, 64, 16, 2048, 8, 256, 1, None) == csa2.ERR_WORKSPACE
    qs[1].w_idx = 16  # weights belong to FP4 keys
    assert g(P(kv), P(sq), qs, 2, 64, 16, 2048, 8, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    # select with appends: at most 8 rows, disjoint storage, rows valid as for csa2_kv_append
    h = L.csa2_index_select_append
    row = lambda layer, lat=None, rp=None, key=None: csa2.AppendRowC(ctypes.pointer(layer), lat, rp, key)
    rows = (csa2.AppendRowC * 2)(row(kv, 16, None, 16), row(kv, 16, None, None))
    assert h(P(kv), P(sq), rows, 2, 16, None, 8, None, 0, 0, 16, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    rows = (csa2.AppendRowC * 1)(row(kv))
    assert h(P(kv), P(sq), rows, 1, 16, None, 8, None, 0, 0, 16, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    rows = (csa2.AppendRowC * 1)(row(rope, 16))  # a rope layer's latent needs its rope row
    assert h(P(kv), P(sq), rows, 1, 16, None, 8, None, 0, 0, 16, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    rows = (csa2.AppendRowC * 1)(row(kv, 16, None, 16))
    assert h(P(kv), P(sq), rows, 9, 16, None, 8, None, 0, 0, 16, 256, 1 << 30, None) == csa2.ERR_INVALID_ARG
    assert h(P(kv), P(sq), rows, 1, 16, None, 8, None, 0, 0, 16, 256, 1, None) == csa2.ERR_WORKSPACE


@needs_lib
def test_noalloc_attention_rejects_before_launch():
    """The allocation-free layered attention checks its arguments and its fixed scratch bound on the host, before
    it resolves the scratch's device address: every case here returns without touching a device."""
    L = csa2.lib()
    P = ctypes.byref
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=None, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    sq = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=1, max_seq_len=64)
    f = L.csa2_sparse_fp4_decode_attn_layers_noalloc
    arr = (csa2.AttnLayerC * 20)(*[csa2.AttnLayerC(ctypes.pointer(kv), 16, 16, 16, None, None, None)
                                   for _ in range(20)])
    assert f(None, 1, P(sq), 64, 64, 0.1, None) == csa2.ERR_INVALID_ARG
    for n_layers, heads, top_k in ((0, 64, 64), (21, 64, 64), (1, 24, 64), (1, 144, 64), (1, 64, 0), (1, 64, 4097)):
        assert f(arr, n_layers, P(sq), heads, top_k, 0.1, None) == csa2.ERR_INVALID_ARG, (n_layers, heads, top_k)
    bad = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=1, max_seq_len=65)
    assert f(arr, 1, P(bad), 64, 64, 0.1, None) == csa2.ERR_INVALID_ARG  # lengths beyond the table
    # 20 layers x 64 sequences x 128 heads: one split's fp32 partials alone (~335 MB) exceed the 32 MiB scratch
    big = csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=64, max_seq_len=64)
    assert f(arr, 20, P(big), 128, 4096, 0.1, None) == csa2.ERR_WORKSPACE
    # the caller-workspace entry point sizes the same problem without refusing it
    n = ctypes.c_size_t()
    assert L.csa2_attn_layers_workspace_size(20, 64, 128, 4096, 512, 0, P(n)) == csa2.OK and n.value > 32 << 20


@needs_lib
def test_batch_bound_rejects_before_launch():
    """At most 65,535 sequences per call (and per layered attention launch, layers x sequences): the largest
    accepted batch passes validation (the call then stops at its missing workspace), one more is refused."""
    L = csa2.lib()
    P = ctypes.byref
    n = ctypes.c_size_t()
    top = 65535
    kv = csa2.KvLayer(codes=16, scales=16, rope=None, idx_keys=16, num_blocks=1, block_tokens=64, latent_dim=512,
                      rope_dim=0, idx_dim=64, idx_dtype=csa2.BF16, idx_heads=1)
    seqs = lambda batch: csa2.Seqs(block_table=16, max_blocks_per_seq=1, seq_lens=16, batch=batch, max_seq_len=64)
    for batch, want_sel, want_size in ((top, csa2.ERR_WORKSPACE, csa2.OK), (top + 1, csa2.ERR_INVALID_ARG,
                                                                            csa2.ERR_INVALID_ARG)):
        sq = seqs(batch)
        assert L.csa2_index_select(P(kv), P(sq), 16, None, 8, csa2.FULL, None, None, 0, 0, 16, 256, 1,
                                   None) == want_sel
        assert L.csa2_sparse_fp4_decode_attn(P(kv), P(sq), 16, 64, 16, 64, 0.1, 16, None, 256, 1,
                                             None) == want_sel
        assert L.csa2_index_select_workspace_size(batch, 64, 8, 0, 8, P(n)) == want_size
        assert L.csa2_attn_workspace_size(batch, 64, 64, 512, P(n)) == want_size
        assert L.csa2_topk_workspace_size(batch, 64, 8, P(n)) == want_size
        assert L.csa2_topk(16, 64, 16, batch, 64, 8, 16, 256, 1, None) == want_sel
    # the layered attention: layers x sequences
    arr = (csa2.AttnLayerC * 3)(*[csa2.AttnLayerC(ctypes.pointer(kv), 16, 16, 16, None, None, None)
                                  for _ in range(3)])
    f = L.csa2_sparse_fp4_decode_attn_layers
    assert f(arr, 3, P(seqs(top // 3)), 64, 64, 0.1, 256, 1, None) == csa2.ERR_WORKSPACE
    assert f(arr, 3, P(seqs(top // 3 + 1)), 64, 64, 0.1, 256, 1, None) == csa2.ERR_INVALID_ARG
    assert L.csa2_attn_layers_workspace_size(3, top // 3, 64, 64, 512, 0, P(n)) == csa2.OK
    assert L.csa2_attn_layers_workspace_size(3, top // 3 + 1, 64, 64, 512, 0, P(n)) == csa2.ERR_INVALID_ARG
    g = L.csa2_sparse_fp4_decode_attn_layers_noalloc
    assert g(arr, 3, P(seqs(top // 3 + 1)), 64, 64, 0.1, None) == csa2.ERR_INVALID_ARG


def test_header_is_plain_c():
    """include/csa2.h is a C header: it compiles as strict C99 and as C++17 (extern "C"), and names no C++,
    HIP or torch type."""
    import shutil
    import subprocess

    hdr = os.path.join(ROOT, "include", "csa2.h")
    for cc, lang, std in (("gcc", "c", "-std=c99"), ("g++", "c++", "-std=c++17")):
        exe = shutil.which(cc)
        if exe is None:
            pytest.skip(f"{cc} not found")
        r = subprocess.run([exe, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", lang, hdr],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    for word in ("torch", "at::", "std::", "hipStream_t", "hip_runtime", "class ", "template"):
        assert word not in text, word


def test_binding_signatures_match_the_header():
    """Every function the header declares has a ctypes signature in the binding with the same number of
    arguments (a missing or extra argument would shift every later one silently)."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "csa2.h")).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    protos = {}
    for m in re.finditer(r"\b(csa2_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", text):
        name, args = m.group(1), m.group(2).strip()
        if name in protos:
            continue
        protos[name] = 0 if args in ("", "void") else args.count(",") + 1
    assert len(protos) >= 25
    for name, nargs in protos.items():
        assert name in csa2.SIGNATURES, f"{name} has no ctypes signature"
        assert len(csa2.SIGNATURES[name][1]) == nargs, (name, nargs, len(csa2.SIGNATURES[name][1]))


def _c_kind(arg):
    """Kind of one C parameter declaration: pointer, 32- or 64-bit integer, size or float."""
    a = arg.strip()
    if "*" in a or re.match(r"(const\s+)?csa2_stream\b", a):
        return "ptr"
    t = a.split()[-2] if len(a.split()) > 1 else a
    return {"int32_t": "i32", "int": "i32", "csa2_mode": "i32", "csa2_dtype": "i32", "csa2_status": "i32", "int64_t": "i64",
            "size_t": "sz", "float": "f32", "uint32_t": "u32"}[t]


def _ctypes_kind(t):
    if t in (ctypes.c_void_p, ctypes.c_char_p) or hasattr(t, "_type_") and isinstance(t._type_, type):
        return "ptr"
    return {ctypes.c_int32: "i32", ctypes.c_int64: "i64", ctypes.c_size_t: "sz", ctypes.c_float: "f32",
            ctypes.c_uint32: "u32"}[t]


def test_binding_argument_kinds_match_the_header():
    """Argument by argument, the ctypes type has the C parameter's kind (a float passed where the header
    takes an int, or a 32-bit count where it takes a 64-bit one, would be read as garbage)."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "csa2.h")).read(), flags=re.S)
    seen = set()
    for m in re.finditer(r"\b(csa2_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", text):
        name, args = m.group(1), m.group(2).strip()
        if name in seen or args in ("", "void"):
            continue
        seen.add(name)
        c = [_c_kind(a) for a in args.split(",")]
        py = [_ctypes_kind(t) for t in csa2.SIGNATURES[name][1]]
        assert c == py, (name, c, py)
    assert len(seen) >= 25


def test_binding_structs_match_the_header_layout():
    """Each ctypes structure of the binding has the size and field offsets the C compiler gives the header's
    struct (a C program built with the host compiler prints them)."""
    import shutil
    import subprocess
    import tempfile

    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    pairs = {"csa2_kv_layer": csa2.KvLayer, "csa2_seqs": csa2.Seqs, "csa2_kv_finish": csa2.KvFinish,
             "csa2_swa_window": csa2.SwaWindow, "csa2_append": csa2.AppendRowC,
             "csa2_reindex_query": csa2.ReindexQueryC, "csa2_attn_layer": csa2.AttnLayerC}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "csa2.h"', "int main(void) {"]
    for cname, cls in pairs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    tmp = tempfile.mkdtemp(prefix="csa2_layout_")
    try:
        src, exe = os.path.join(tmp, "layout.c"), os.path.join(tmp, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        r = subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", exe, src], capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        out = subprocess.run([exe], capture_output=True, text=True, timeout=60).stdout.split("\n")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    got = {}
    for line in out:
        if line:
            cname, key, val = line.split()
            got[(cname, key)] = int(val)
    for cname, cls in pairs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert got[(cname, field)] == getattr(cls, field).offset, (cname, field)


def test_launch_timer_accepts_every_documented_name():
    """csa2_time_next_launch arms for each kernel name the header lists (and for every name bench.py times),
    refuses others, and disarms with NULL; arming launches nothing."""
    L = csa2.lib()
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    block = text[text.index("Profiling aid"):text.index("csa2_status csa2_time_next_launch")]
    names = re.findall(r'"([a-z_0-9]+)"', block)
    assert len(names) >= 8
    bench = open(os.path.join(ROOT, "bench.py")).read()
    timed = set(re.findall(r'kernel_ms\("([a-z_]+)"', bench)) | set(re.findall(r'"([a-z_]+)": "[a-z]+\.hip"', bench))
    assert timed and timed <= set(names), timed - set(names)
    ev = ctypes.c_void_p(16)
    for name in names:
        assert L.csa2_time_next_launch(name.encode(), ev, ev) == csa2.OK, name
        assert L.csa2_timer_pending() == 1
        assert L.csa2_time_next_launch(None, None, None) == csa2.OK
        assert L.csa2_timer_pending() == 0
    assert L.csa2_time_next_launch(b"no_such_kernel", ev, ev) == csa2.ERR_INVALID_ARG
    assert L.csa2_timer_pending() == 0


def test_build_compiles_every_hip_source():
    """The build compiles every .hip file under csrc (a source left out of the list would drop its kernels
    from the library without a compile error)."""
    from sparse_attention_fp4_kv_amd import build_lib

    on_disk = sorted(os.path.basename(p) for p in glob.glob(os.path.join(build_lib.CSRC, "*.hip")))
    assert sorted(build_lib.SOURCES) == on_disk
