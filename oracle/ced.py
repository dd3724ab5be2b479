"""CED global-KV projection of the oracle.

Source: [P1] section "Causal Encoder-Decoder": for every decoder layer l > L/2
the global KV is projected from the last encoder hidden state H_{L/2} with
per-layer weights, C_l = H_{L/2} W_l^KV and Z_l = H_{L/2} W_l^Z.  [P3]
"규모와 구조" and [P4] section 2 restate the 20 + 20 split.

Readings taken where the pages are silent:
  * Z_l is the indexer key of layer l (64 channels); C_l is the 512-channel
    main-KV latent that is then stored in the FP4 format.
  * No normalisation or rotary step is applied between the projection and the
    pack (the formula is taken literally).
  * Weights are stored in the out x in orientation (W^T, as a Linear layer
    stores them): w_kv[l] is [512][hidden], w_z[l] is [64][hidden].
  * Z is stored in bf16, rounded to nearest-even from the exact product.

Parity pins (tests/test_oracle_ced.py): permutation-matrix weights select
(and reorder) channels of H exactly, which catches transposed or swapped
operands and a wrong layer index; a pure-Python triple loop on a tiny case;
the bf16 rounding of Z against torch's float32 -> bfloat16 conversion on
values where float32 is exact.
"""

import numpy as np

from . import fp4


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 (nearest, ties to even) -> uint16 bits.

    The value is first split exactly into its fp32 neighbourhood: rounding a
    float64 straight to 8 significant bits is done on the float64 mantissa so
    there is no double rounding through fp32.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                # 8 significant bits to the left of the point
    r = np.round(scaled)                   # numpy rounds half to even
    y = np.ldexp(r, e - 8)                 # exact in fp32 range for our inputs
    out = y.astype(np.float32)
    return (out.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def ced_project(h_bits, w_kv_bits, w_z_bits=None):
    """C_l and Z_l for all layers in float64.

    h_bits:    uint16 bf16 [T][hidden]
    w_kv_bits: uint16 bf16 [L][512][hidden]   (out x in)
    w_z_bits:  uint16 bf16 [L][64][hidden] or None
    returns (C float64 [L][T][512], Z float64 [L][T][64] or None)
    """
    H = bf16_bits_to_f64(h_bits)
    Wkv = bf16_bits_to_f64(w_kv_bits)
    C = np.stack([H @ Wkv[l].T for l in range(Wkv.shape[0])])
    Z = None
    if w_z_bits is not None:
        Wz = bf16_bits_to_f64(w_z_bits)
        Z = np.stack([H @ Wz[l].T for l in range(Wz.shape[0])])
    return C, Z


def ced_project_and_pack(h_bits, w_kv_bits, w_z_bits=None):
    """The full CED output as stored: FP4 (codes, scales) of C and bf16 Z.

    C is rounded to fp32 (the accumulator precision of the stored latent)
    before packing.  returns codes uint8 [L][T][256], scales uint8 [L][T][32],
    z uint16 [L][T][64] or None, and the float64 C for tolerance checks.
    """
    C, Z = ced_project(h_bits, w_kv_bits, w_z_bits)
    codes, scales = fp4.fp4_pack(C.astype(np.float32))
    z = f64_to_bf16_bits(Z) if Z is not None else None
    return codes, scales, z, C
