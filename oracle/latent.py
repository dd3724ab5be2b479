"""Finishing a KV latent before it is cached, and the indexer key taken from it (oracle).

Sources:
  [P1] section "FP4 KV cache": the range argument for dropping NVFP4's global
       scale says the 512-channel KV latent is RMS-normalised (learned weight
       of magnitude about 1, so its L2 norm stays near sqrt(512)) and then
       rotated by RoPE, which keeps the norm; the result is what the FP4 pack
       stores.
  [P1] section "CSA2" (mode table and the paragraph after it): a Full layer
       obtains its indexer K by projecting the main KV rather than through a
       separate path from the hidden state; the indexer has 32 query heads of
       dimension 128.

Readings taken where the pages are silent (each is listed in the design notes):
  * RMSNorm: y_j = x_j / sqrt(mean_j x_j^2 + eps) * gamma_j over the 512
    channels, eps and gamma given by the caller.
  * RoPE acts on the last 64 channels (448 .. 511), the width of the
    positional part in DeepSeek's attention, in adjacent pairs
    (448 + 2i, 449 + 2i), i = 0 .. 31: (a, b) -> (a cos t - b sin t,
    a sin t + b cos t) with t = p * theta^(-2i / 64) at token position p.
    The angle is formed the way fp32 inference code forms it: the frequency
    fl32(theta^(-2i/64)) and the product fl32(p * frequency) are fp32 values;
    cos and sin of that fp32 angle are then exact (float64 here).
    theta == 0 means no rotation.
  * The indexer key is the projection of the cached entry: k = W_idx x_hat,
    where x_hat is the dequantized FP4 latent (what Reindex and Reuse layers
    find in the cache) and W_idx is a bf16 [128][512] weight (out x in); the
    key is then stored in the same FP4 format (V4 already kept indexer keys in
    FP4).

Parity pins (tests/test_oracle_latent.py): RMSNorm of a constant vector and
its scale invariance; RoPE at p = 0 is the identity, keeps every pair's norm,
rotates by a hand-computed angle, and keeps q.k a function of the position
difference only; with gamma = 1, no rotation and an input of RMS exactly 1 the
finished entry is the plain pack of the input; a permutation-matrix W_idx picks
channels of the dequantized entry exactly.
"""

import numpy as np

from . import fp4

LATENT = 512
ROPE_DIMS = 64
ROPE_FIRST = LATENT - ROPE_DIMS
IDX_DIM = 128


def rms_norm(x, gamma, eps):
    """x [..., 512] -> x / sqrt(mean(x^2) + eps) * gamma, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)


def rope_frequencies(theta):
    """fp32 frequencies theta^(-2i/64), i = 0 .. 31 (rounded once from float64)."""
    i = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    return (float(theta) ** (-2.0 * i / ROPE_DIMS)).astype(np.float32)


def rope_angles(positions, theta):
    """fp32 angles fl32(p * f_i): [n][32] for integer positions [n]."""
    p = np.asarray(positions, dtype=np.int64).astype(np.float32)
    return (p[:, None] * rope_frequencies(theta)[None, :]).astype(np.float32)


def rope(x, positions, theta):
    """Rotate channels 448 .. 511 of x [n][512] in adjacent pairs by the angles of `positions` [n]."""
    y = np.array(x, dtype=np.float64, copy=True)
    if theta == 0:
        return y
    t = rope_angles(positions, theta).astype(np.float64)
    c, s = np.cos(t), np.sin(t)
    a = y[:, ROPE_FIRST::2].copy()
    b = y[:, ROPE_FIRST + 1::2].copy()
    y[:, ROPE_FIRST::2] = a * c - b * s
    y[:, ROPE_FIRST + 1::2] = a * s + b * c
    return y


def finish_latent(c, positions, gamma, eps, theta):
    """Raw latents c [n][512] -> the entry before packing (RMSNorm, then RoPE), float64."""
    return rope(rms_norm(c, gamma, eps), positions, theta)


def indexer_key(codes, scales, w_idx_bits):
    """k = W_idx x_hat for cached entries (codes [n][256], scales [n][32]); W_idx bf16 bits [128][512]."""
    from .ced import bf16_bits_to_f64

    x_hat = fp4.fp4_unpack(codes, scales)
    return x_hat @ bf16_bits_to_f64(w_idx_bits).T


def kv_entry(c, positions, gamma, eps, theta, w_idx_bits=None):
    """The whole chain for raw latents c [n][512] at `positions`.

    Returns (x float64 [n][512] before packing, codes, scales, k float64 [n][128] or None,
    k_codes, k_scales).  The pack takes its decisions on fp32 inputs, so x is
    rounded to fp32 before packing (the kernel packs fp32 values), and so is k.
    """
    x = finish_latent(c, positions, gamma, eps, theta)
    codes, scales = fp4.fp4_pack(x.astype(np.float32))
    if w_idx_bits is None:
        return x, codes, scales, None, None, None
    k = indexer_key(codes, scales, w_idx_bits)
    kc, ks = fp4.fp4_pack(k.astype(np.float32))
    return x, codes, scales, k, kc, ks
