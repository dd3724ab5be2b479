"""GPU parity of the CED projection with the fused FP4 pack."""

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

from _util import pack_close, to_dev

pytestmark = pytest.mark.gpu


def _bits(x):
    return wl.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_identity_weights_bit_exact():
    """hidden = 512, W_kv = I: C = H exactly, so the fused pack equals the oracle pack of H."""
    rng = np.random.default_rng(0)
    T = 300  # ragged against the 256-row tile
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


@pytest.mark.parametrize("hidden,T", [(64, 1), (128, 257), (192, 513)])
def test_integer_weights_short_k_and_ragged_rows(hidden, T):
    """The shortest reductions (2, 4 and 6 k-steps of 32: the load pipeline's start-up and drain without a
    steady state) and row counts of 1, one past a 256-row tile and one past two, with W^Z: exact as above."""
    rng = np.random.default_rng(2 + hidden)
    L = 2
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


def _check_ced_rows(codes, scales, z, c, h, wkv, wz, hidden):
    """Sampled rows of one CED call against the oracle (every array holds the same rows):
      * C (fp32 accumulators) within hidden * 2^-24 * sum|H||W| of the float64 product
        (the standard bound of a length-`hidden` fp32 sum of exact bf16 products);
      * the fused pack equals the oracle's pack of the GPU's own fp32 C, bit for bit;
      * against the oracle's pack of the exact C, a group differs only where an element or
        the group's amax lies within that C bound of a decision point (pack_close);
      * Z is the bf16 rounding (half an ulp: 2^-8 relative) of an fp32 sum within the same
        kind of bound of the exact Z_l = H W_l^Z:  |Z_gpu - Z| <= 2^-8 (|Z| + b) + b,
        b = hidden * 2^-24 * sum|H||W_z|.
    Returns the number of groups that differ from the oracle's pack of the exact C."""
    L = wkv.shape[0]
    C, Z = oracle.ced.ced_project(h, wkv, wz)
    H = np.abs(oracle.ced.bf16_bits_to_f64(h))
    W = np.abs(oracle.ced.bf16_bits_to_f64(wkv))
    bound = np.stack([H @ W[l].T for l in range(L)]) * hidden * 2.0 ** -24
    cg = c.astype(np.float64)
    assert np.all(np.abs(cg - C) <= bound)
    diff = 0
    for l in range(L):
        oc, os_ = oracle.fp4.fp4_pack(c[l])
        assert np.array_equal(codes[l], oc), f"layer {l}: fused codes differ from the oracle pack of C"
        assert np.array_equal(scales[l], os_), f"layer {l}: fused scales differ from the oracle pack of C"
        diff += pack_close(codes[l], scales[l], C[l], rel=0.0, abs_=0.0, tol=bound[l])
    zz = oracle.ced.bf16_bits_to_f64(z.view(np.uint16))
    Wz = np.abs(oracle.ced.bf16_bits_to_f64(wz))
    bound_z = np.stack([H @ Wz[l].T for l in range(L)]) * hidden * 2.0 ** -24
    assert np.all(np.abs(zz - Z) <= 2.0 ** -8 * (np.abs(Z) + bound_z) + bound_z)
    return diff


@pytest.mark.parametrize("hidden", [4096, 5120])
def test_random_within_fp32_bound(hidden):
    """Random bf16 inputs (hidden 4096, and the model's 5120), every row checked as _check_ced_rows says."""
    st = wl.Streams(3)
    T, L = 384, 2
    h, wkv, wz = wl.ced_inputs(st, T, hidden, L)
    codes, scales, z, c = csa2.csa2_ced_kv_project(to_dev(h), to_dev(wkv), to_dev(wz), c_f32=True)
    torch.cuda.synchronize()
    _check_ced_rows(codes.cpu().numpy(), scales.cpu().numpy(), z.cpu().numpy(), c.cpu().numpy(), h, wkv, wz,
                    hidden)


def test_full_prefill_shape_sampled_rows():
    """The 16,384-token x 4096 prefill into 20 layers (512 FP4 + 64 bf16 each), the bench's own call and
    launch shape (64 row tiles x 90 column tiles, XCD-remapped groups).  Every layer is checked on 320
    seeded rows (256 random, the first and last 32 of the sequence) as _check_ced_rows says; the call
    without the fp32 copy of C (as the bench times it) writes the same bytes."""
    st = wl.Streams(3)
    T, hidden, L = 16384, 4096, 20
    h, wkv, wz = wl.ced_inputs(st, T, hidden, L)
    h_d, wkv_d, wz_d = to_dev(h), to_dev(wkv), to_dev(wz)
    codes, scales, z, c = csa2.csa2_ced_kv_project(h_d, wkv_d, wz_d, c_f32=True)
    codes2, scales2, z2, _ = csa2.csa2_ced_kv_project(h_d, wkv_d, wz_d)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2) and torch.equal(z, z2)
    del codes2, scales2, z2
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([rng.choice(T, 256, replace=False), np.arange(32), np.arange(T - 32, T)]))
    r_d = torch.from_numpy(rows).to(codes.device)
    pick = lambda t: t[:, r_d].cpu().numpy()
    diff = _check_ced_rows(pick(codes), pick(scales), pick(z), pick(c), h[rows], wkv, wz, hidden)
    assert diff <= 0.01 * L * len(rows) * 32, diff  # differences from the exact C are rare
