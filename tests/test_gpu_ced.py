"""GPU parity of the CED projection with the fused FP4 pack."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import to_dev

pytestmark = pytest.mark.gpu


def _bits(x):
    return wl.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_identity_weights_bit_exact():
    """hidden = 512, W_kv = I: C = H exactly, so the fused pack equals the oracle pack of H."""
    rng = np.random.default_rng(0)
    T = 300  # ragged against the 128-row tile
    h = _bits(rng.standard_normal((T, 512)) * 4)
    w = np.broadcast_to(np.eye(512, dtype=np.float32), (2, 512, 512))
    codes, scales, z, c = csa2.csa2_ced_kv_project(to_dev(h), to_dev(_bits(w)), c_f32=True)
    torch.cuda.synchronize()
    hc = oracle.ced.bf16_bits_to_f64(h).astype(np.float32)
    oc, os_ = oracle.fp4.fp4_pack(hc)
    for l in range(2):
        assert np.array_equal(codes[l].cpu().numpy(), oc)
        assert np.array_equal(scales[l].cpu().numpy(), os_)
        assert np.array_equal(c[l].cpu().numpy(), hc)


def test_integer_weights_exact_all_outputs():
    """Small integers: every product and sum is exact in fp32, so C, packed C and Z are exact."""
    rng = np.random.default_rng(1)
    T, hidden, L = 200, 256, 3
    h = _bits(rng.integers(-3, 4, size=(T, hidden)))
    wkv = _bits(rng.integers(-2, 3, size=(L, 512, hidden)))
    wz = _bits(rng.integers(-2, 3, size=(L, 64, hidden)))
    codes, scales, z, c = csa2.csa2_ced_kv_project(to_dev(h), to_dev(wkv), to_dev(wz), c_f32=True)
    torch.cuda.synchronize()
    oc, os_, oz, C = oracle.ced.ced_project_and_pack(h, wkv, wz)
    assert np.array_equal(c.cpu().numpy(), C.astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(z.cpu().numpy().view(np.uint16), oz)


@pytest.mark.parametrize("hidden", [4096, 5120])
def test_random_within_fp32_bound(hidden):
    """Random bf16 inputs (hidden 4096, and the model's 5120): fp32 C within hidden * 2^-24 *
    sum|H||W| of the fp64 C; packed bytes may differ from the oracle's only where the value
    sits within that bound of a decision threshold; Z within one bf16 ulp."""
    st = wl.Streams(3)
    T, L = 384, 2
    h, wkv, wz = wl.ced_inputs(st, T, hidden, L)
    codes, scales, z, c = csa2.csa2_ced_kv_project(to_dev(h), to_dev(wkv), to_dev(wz), c_f32=True)
    torch.cuda.synchronize()
    C, Z = oracle.ced.ced_project(h, wkv, wz)
    H = np.abs(oracle.ced.bf16_bits_to_f64(h))
    W = np.abs(oracle.ced.bf16_bits_to_f64(wkv))
    bound = np.stack([H @ W[l].T for l in range(L)]) * hidden * 2.0 ** -24
    cg = c.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(cg - C) <= bound)
    # the fused pack of the GPU's fp32 C equals the standalone GPU pack of that C
    c2, s2 = csa2.csa2_fp4_pack(c.reshape(-1, 512))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().reshape(-1, 256), c2.cpu().numpy())
    assert np.array_equal(scales.cpu().numpy().reshape(-1, 32), s2.cpu().numpy())
    # against the oracle's pack of the exact C: differences only near decision points
    oc, os_ = oracle.fp4.fp4_pack(C.astype(np.float32))
    gs = scales.cpu().numpy()
    frac = np.mean(gs != os_)
    assert frac < 1e-3, frac
    # Z: bf16 rounding (half an ulp, 2^-8 relative) of an fp32 sum that is itself
    # within the accumulation bound of the exact value
    zz = oracle.ced.bf16_bits_to_f64(z.cpu().numpy().view(np.uint16))
    Wz = np.abs(oracle.ced.bf16_bits_to_f64(wz))
    bound_z = np.stack([H @ Wz[l].T for l in range(L)]) * hidden * 2.0 ** -24
    assert np.all(np.abs(zz - Z) <= 2.0 ** -8 * (np.abs(Z) + bound_z) + bound_z)
