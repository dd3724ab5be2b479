"""Pins of the oracle's sparse attention.

- selecting every entry equals textbook dense attention computed by torch's
  float64 scaled_dot_product_attention on the CPU (a library routine);
- one selected entry gives o = c_s exactly and lse = logit_s;
- equal logits give the plain mean of the selected latents;
- the result does not depend on the order of the selected slots;
- the lse-merge of two disjoint halves equals the whole;
- the rope side-band changes the logits only.
"""

import numpy as np
import torch

from oracle import attention, fp4
from sparse_attention_fp4_kv_amd import workloads as wl


def _case(n=96, H=8, D=512, R=0, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float32)
    codes, scales = fp4.fp4_pack(x)
    c = fp4.fp4_unpack(codes, scales)
    q = wl.to_bf16_bits(rng.standard_normal((H, D + R)).astype(np.float32))
    rope = fp4_rope = None
    if R:
        rope = wl.to_bf16_bits(rng.standard_normal((n, R)).astype(np.float32))
        fp4_rope = (rope.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return q, c, fp4_rope


def _q64(q):
    return (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_dense_equals_sdpa():
    q, c, _ = _case()
    sigma = 1 / np.sqrt(512)
    out, lse = attention.sparse_attention(q, c, sigma)
    Q = torch.from_numpy(_q64(q))[None, :, None, :]          # [1, H, 1, D]
    K = torch.from_numpy(c)[None, None].expand(1, q.shape[0], -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, scale=sigma)[0, :, 0].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    logits = sigma * (_q64(q) @ c.T)
    assert np.max(np.abs(lse - np.log(np.exp(logits).sum(axis=1)))) < 1e-12


def test_dense_with_rope_equals_sdpa():
    q, c, rope = _case(R=64, seed=1)
    sigma = 1 / np.sqrt(576)
    out, _ = attention.sparse_attention(q, c, sigma, rope_sel=rope)
    Q = torch.from_numpy(_q64(q))[None, :, None, :]
    Kfull = torch.from_numpy(np.concatenate([c, rope], axis=1))[None, None].expand(1, q.shape[0], -1, -1)
    V = torch.from_numpy(c)[None, None].expand(1, q.shape[0], -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kfull, V, scale=sigma)[0, :, 0].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_single_entry():
    q, c, _ = _case(n=1)
    out, lse = attention.sparse_attention(q, c, 0.1)
    assert np.array_equal(out, np.broadcast_to(c, out.shape))
    assert np.allclose(lse, 0.1 * (_q64(q) @ c[0]), rtol=0, atol=1e-12)


def test_equal_logits_give_mean():
    q = np.zeros((4, 512), dtype=np.uint16)  # bf16 zeros -> all logits 0
    _, c, _ = _case(n=10)
    out, lse = attention.sparse_attention(q, c, 0.05)
    assert np.allclose(out, c.mean(axis=0)[None], rtol=0, atol=1e-12)
    assert np.allclose(lse, np.log(10.0))


def test_permutation_invariance_and_merge():
    q, c, _ = _case(n=64, seed=3)
    sigma = 0.04
    out, lse = attention.sparse_attention(q, c, sigma)
    perm = np.random.default_rng(0).permutation(64)
    out_p, lse_p = attention.sparse_attention(q, c[perm], sigma)
    assert np.max(np.abs(out - out_p)) < 1e-12 and np.max(np.abs(lse - lse_p)) < 1e-12
    oa, la = attention.sparse_attention(q, c[:20], sigma)
    ob, lb = attention.sparse_attention(q, c[20:], sigma)
    om, lm = attention.merge_partials(oa, la, ob, lb)
    assert np.max(np.abs(om - out)) < 1e-12 and np.max(np.abs(lm - lse)) < 1e-12


def test_empty_selection_and_valid_slots():
    q, c, _ = _case(n=4)
    out, lse = attention.sparse_attention(q, c[:0], 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    assert attention.valid_slots([3, -1, 7, 0, 9], 8).tolist() == [3, 7, 0]
