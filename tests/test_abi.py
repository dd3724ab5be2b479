"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and its host-side validation and page allocator behave as
documented (no GPU work is launched by any call here)."""

import ctypes
import os
import re

import pytest

from sparse_attention_fp4_kv_amd import csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAVE_LIB = os.path.exists(csa2.LIB_PATH)
needs_lib = pytest.mark.skipif(not HAVE_LIB, reason="libcsa2.so not built")


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
    assert csa2.lib().csa2_abi_version() == 5
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
