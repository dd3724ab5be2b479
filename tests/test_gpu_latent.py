"""GPU parity of the latent finish (RMSNorm, RoPE, FP4 pack) and of the FP4 indexer key projected from
the cached entry: rows mode, the CED projection with the finish, and the finishing append."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import build_tables, make_batch, pack_close, to_dev

pytestmark = pytest.mark.gpu

EPS, THETA = 1e-6, 10000.0


def _inputs(seed, L, T):
    st = wl.Streams(seed)
    c = np.stack([wl.latent_rows(st, l, 0, T) for l in range(L)]) * np.float32(0.7)
    gamma, w_idx = wl.kv_finish_inputs(st, L)
    return c, gamma, w_idx


@pytest.mark.parametrize("pos0", [0, 1000, (1 << 24) - 300])
def test_finish_rows_match_oracle(pos0):
    L, T = 2, 300  # ragged against the 32-row workgroup
    c, gamma, w_idx = _inputs(80, L, T)
    codes, scales, kc, ks, x, k = csa2.csa2_kv_finish_rows(to_dev(c), to_dev(gamma), EPS, THETA, to_dev(w_idx),
                                                           pos0=pos0, debug=True)
    torch.cuda.synchronize()
    codes, scales, kc, ks = (t.cpu().numpy() for t in (codes, scales, kc, ks))
    x, k = x.cpu().numpy(), k.cpu().numpy()
    # the packs of the GPU's own fp32 values are the standalone pack's (itself bit-exact with the oracle)
    p_c, p_s = csa2.csa2_fp4_pack(to_dev(x.reshape(-1, 512)))
    q_c, q_s = csa2.csa2_fp4_pack(to_dev(k.reshape(-1, 128)))
    torch.cuda.synchronize()
    assert np.array_equal(codes.reshape(-1, 256), p_c.cpu().numpy())
    assert np.array_equal(scales.reshape(-1, 32), p_s.cpu().numpy())
    assert np.array_equal(kc.reshape(-1, 64), q_c.cpu().numpy())
    assert np.array_equal(ks.reshape(-1, 8), q_s.cpu().numpy())
    pos = pos0 + np.arange(T)
    total_rows, key_rows, diff_groups = 0, 0, 0
    for l in range(L):
        xr, oc, os_, kr, okc, oks = oracle.latent.kv_entry(c[l], pos, gamma[l], EPS, THETA, w_idx[l])
        # fp32 chain: sum of squares, correctly rounded sqrt / divide, fp32 sin / cos of the shared fp32 angle
        assert np.all(np.abs(x[l] - xr) <= 4e-6 * (1.0 + np.abs(xr))), float(np.max(np.abs(x[l] - xr)))
        diff_groups += pack_close(codes[l], scales[l], xr, rel=4e-6, abs_=4e-6)
        # the key: rows whose entry bytes equal the oracle's are compared with the oracle's key
        same = np.all(codes[l] == oc, axis=1) & np.all(scales[l] == os_, axis=1)
        total_rows += T
        key_rows += int(same.sum())
        xh = np.abs(oracle.fp4.fp4_unpack(oc, os_))
        bound = 512 * 2.0 ** -24 * (xh @ np.abs(oracle.ced.bf16_bits_to_f64(w_idx[l])).T)
        assert np.all(np.abs(k[l][same] - kr[same]) <= bound[same])
        pack_close(kc[l][same], ks[l][same], kr[same], rel=1e-6, abs_=float(bound[same].max()))
    assert diff_groups <= 1e-3 * total_rows * 32, diff_groups
    assert key_rows >= 0.95 * total_rows, (key_rows, total_rows)


def test_finish_exact_case():
    """gamma on a coarse grid, entries +-1 (mean square exactly 1, eps far below an ulp), position 0 (the
    rotation is the identity) and a permutation W_idx: every output byte equals the oracle's."""
    rng = np.random.default_rng(81)
    L, T = 1, 70
    c = rng.choice([-1.0, 1.0], size=(L, T, 512)).astype(np.float32)
    gamma = (rng.integers(8, 65, size=(L, 512)) / 64.0).astype(np.float32)
    sel = rng.permutation(512)[:128]
    w = np.zeros((L, 128, 512), dtype=np.float32)
    w[0, np.arange(128), sel] = 1.0
    w_bits = wl.to_bf16_bits(w)
    codes, scales, kc, ks, _, _ = csa2.csa2_kv_finish_rows(to_dev(c[:, :1]), to_dev(gamma), 1e-30, THETA,
                                                           to_dev(w_bits))
    torch.cuda.synchronize()
    x, oc, os_, k, okc, oks = oracle.latent.kv_entry(c[0, :1], [0], gamma[0], 1e-30, THETA, w_bits[0])
    assert np.array_equal(codes.cpu().numpy()[0], oc) and np.array_equal(scales.cpu().numpy()[0], os_)
    assert np.array_equal(kc.cpu().numpy()[0], okc) and np.array_equal(ks.cpu().numpy()[0], oks)
    # no rotation: every position is exact
    codes, scales, kc, ks, _, _ = csa2.csa2_kv_finish_rows(to_dev(c), to_dev(gamma), 1e-30, 0.0, to_dev(w_bits),
                                                           pos0=12345)
    torch.cuda.synchronize()
    x, oc, os_, k, okc, oks = oracle.latent.kv_entry(c[0], np.arange(T), gamma[0], 1e-30, 0.0, w_bits[0])
    assert np.array_equal(codes.cpu().numpy()[0], oc) and np.array_equal(scales.cpu().numpy()[0], os_)
    assert np.array_equal(kc.cpu().numpy()[0], okc) and np.array_equal(ks.cpu().numpy()[0], oks)


def test_ced_project_finished_is_projection_then_finish():
    st = wl.Streams(82)
    T, hidden, L = 200, 1024, 3
    h, wkv, _ = wl.ced_inputs(st, T, hidden, L)
    gamma, w_idx = wl.kv_finish_inputs(st, L)
    codes, scales, kc, ks, c = csa2.csa2_ced_kv_project_finished(to_dev(h), to_dev(wkv), to_dev(gamma), EPS, THETA,
                                                                  to_dev(w_idx), pos0=77)
    _, _, _, c_ref = csa2.csa2_ced_kv_project(to_dev(h), to_dev(wkv), c_f32=True)
    f = csa2.csa2_kv_finish_rows(c_ref, to_dev(gamma), EPS, THETA, to_dev(w_idx), pos0=77)
    torch.cuda.synchronize()
    assert torch.equal(c, c_ref)
    for a, b in zip((codes, scales, kc, ks), f[:4]):
        assert torch.equal(a, b)
    # and the projection itself against the oracle's exact product
    C, _ = oracle.ced.ced_project(h, wkv, None)
    H = np.abs(oracle.ced.bf16_bits_to_f64(h))
    W = np.abs(oracle.ced.bf16_bits_to_f64(wkv))
    bound = np.stack([H @ W[l].T for l in range(L)]) * hidden * 2.0 ** -24
    assert np.all(np.abs(c.cpu().numpy().astype(np.float64) - C) <= bound)


def test_append_finished_matches_rows_at_the_slot():
    st = wl.Streams(83)
    seq_lens = [63, 64, 0, 130, 5000, 70]
    B = len(seq_lens)
    tables, nb = build_tables(st, seq_lens, True, extra_blocks=1)
    tables[5, :] = -1  # sequence 5 has no page: skipped
    layer = csa2.PagedLayer(nb, idx_dtype="fp4", device="cuda")
    batch = make_batch(tables, seq_lens)
    c = wl.latent_rows(st, 0, 1, B) * np.float32(0.5)
    gamma, w_idx = wl.kv_finish_inputs(st, 1)
    csa2.csa2_kv_append_finished(layer, batch, to_dev(c), to_dev(gamma[0]), EPS, THETA, to_dev(w_idx[0]))
    torch.cuda.synchronize()
    gc, gs = layer.codes.cpu().numpy(), layer.scales.cpu().numpy()
    gk, gks = layer.idx_keys.cpu().numpy(), layer.idx_scales.cpu().numpy()
    written = []
    for b, n in enumerate(seq_lens):
        f = csa2.csa2_kv_finish_rows(to_dev(c[b:b + 1][None]), to_dev(gamma), EPS, THETA, to_dev(w_idx), pos0=n)
        torch.cuda.synchronize()
        if b == 5:
            continue
        row = int(oracle.paged.physical_rows(tables[b], np.array([n]))[0])
        written.append(row)
        assert np.array_equal(gc[row], f[0].cpu().numpy()[0, 0]) and np.array_equal(gs[row], f[1].cpu().numpy()[0, 0])
        assert np.array_equal(gk[row], f[2].cpu().numpy()[0, 0]) and np.array_equal(gks[row], f[3].cpu().numpy()[0, 0])
        # and against the oracle chain at that position
        xr, oc, os_, kr, okc, oks = oracle.latent.kv_entry(c[b:b + 1], [n], gamma[0], EPS, THETA, w_idx[0])
        pack_close(gc[row:row + 1], gs[row:row + 1], xr, rel=4e-6, abs_=4e-6)
    others = np.setdiff1d(np.arange(gc.shape[0]), written)
    assert not gc[others].any() and not gs[others].any() and not gk[others].any() and not gks[others].any()


def test_finish_rows_without_key_projection():
    """Without W_idx only the entry is written, and it is the same entry as with the key."""
    L, T = 2, 70
    c, gamma, w_idx = _inputs(84, L, T)
    a = csa2.csa2_kv_finish_rows(to_dev(c), to_dev(gamma), EPS, THETA, None, pos0=5)
    b = csa2.csa2_kv_finish_rows(to_dev(c), to_dev(gamma), EPS, THETA, to_dev(w_idx), pos0=5)
    torch.cuda.synchronize()
    assert a[2] is None and a[3] is None
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
