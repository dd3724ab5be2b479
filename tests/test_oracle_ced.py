"""Pins of the oracle's CED projection.

- permutation-matrix weights: C_l must be H with its channels reordered by the
  layer's own permutation, exactly; this fails for a transposed weight, a
  swapped operand or a wrong layer index;
- a pure-Python triple loop on a tiny case;
- the bf16 rounding of Z against torch's float32 -> bfloat16 conversion on
  values that are exact in float32, and ties-to-even cases worked by hand;
- with W = I (hidden = 512) the packed C is the pack of H itself.
"""

import numpy as np
import torch

from oracle import ced, fp4
from sparse_attention_fp4_kv_amd import workloads as wl


def _bits(x):
    return wl.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_permutation_weights_select_channels():
    rng = np.random.default_rng(0)
    T, hidden, L = 7, 600, 3
    H = rng.standard_normal((T, hidden)).astype(np.float32)
    Hb = _bits(H)
    Hf = ced.bf16_bits_to_f64(Hb)
    W = np.zeros((L, 512, hidden), dtype=np.float32)
    Wz = np.zeros((L, 64, hidden), dtype=np.float32)
    perms = [rng.permutation(hidden)[:512] for _ in range(L)]
    zperms = [rng.permutation(hidden)[:64] for _ in range(L)]
    for l in range(L):
        W[l, np.arange(512), perms[l]] = 1.0      # out channel o reads input perms[l][o]
        Wz[l, np.arange(64), zperms[l]] = 2.0
    C, Z = ced.ced_project(Hb, _bits(W), _bits(Wz))
    for l in range(L):
        assert np.array_equal(C[l], Hf[:, perms[l]])
        assert np.array_equal(Z[l], 2.0 * Hf[:, zperms[l]])


def test_triple_loop_tiny():
    rng = np.random.default_rng(1)
    T, hidden, L = 3, 16, 2
    Hb = _bits(rng.standard_normal((T, hidden)))
    Wb = _bits(rng.standard_normal((L, 512, hidden)))
    C, _ = ced.ced_project(Hb, Wb)
    Hf, Wf = ced.bf16_bits_to_f64(Hb), ced.bf16_bits_to_f64(Wb)
    for l in range(L):
        for t in range(T):
            for o in (0, 1, 255, 511):
                acc = 0.0
                for k in range(hidden):
                    acc += Hf[t, k] * Wf[l, o, k]
                assert abs(acc - C[l, t, o]) <= 1e-12 * (1 + abs(acc))


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(5000) * np.exp(rng.uniform(-10, 10, 5000))).astype(np.float32)
    ours = ced.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_by_hand():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins.
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even (1 + 2^-6) wins.
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40])
    got = ced.f64_to_bf16_bits(vals)
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F81]


def test_identity_weights_reduce_to_pack():
    rng = np.random.default_rng(3)
    T = 9
    Hb = _bits(rng.standard_normal((T, 512)) * 3)
    W = np.eye(512, dtype=np.float32)[None]
    codes, scales, z, C = ced.ced_project_and_pack(Hb, _bits(W))
    c_ref, s_ref = fp4.fp4_pack(ced.bf16_bits_to_f64(Hb).astype(np.float32))
    assert np.array_equal(codes[0], c_ref) and np.array_equal(scales[0], s_ref)
    assert z is None
