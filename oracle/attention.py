"""Sparse FP4 decode attention of the oracle.

Sources:
  [P1] section "CSA2": KV cost is cut on three axes at once; on the entry-size
       axis a small latent vector is shared by all heads (MLA style), and the
       attention of a layer reads only its top-K selected entries.
  [P1] section "FP4 KV cache": cache values are dequantized before attention.
  [P4] section 2: 64 attention heads, 1 KV head.

Readings taken where the pages are silent:
  * K = V = the dequantized 512-channel latent, shared by every head.  An
    optional rope side-band (bf16, 64 dims) takes part in the logits only.
  * logit_s = sigma * (q[:512] . c_s + q[512:] . rope_s); o = softmax-weighted
    sum of c_s; lse = log-sum-exp of the logits.  sigma is the caller's.
  * Selected slots that are -1 or >= the sequence length are skipped; an
    empty selection gives o = 0 and lse = -inf.
  * The query is bf16; the arithmetic here is float64.

Parity pins (tests/test_oracle_attention.py): K = n against torch's float64
scaled_dot_product_attention on the dequantized cache; |S| = 1 gives o = c_s
and lse = logit_s exactly; equal logits give the mean; invariance under a
permutation of the selected slots; lse-merge of two halves of S.
"""

import numpy as np

from .ced import bf16_bits_to_f64


def sparse_attention(q_bits, c_sel, sigma, rope_sel=None):
    """Attention of H query heads over the selected entries.

    q_bits:   uint16 bf16 [H][D (+R)]
    c_sel:    float64 [S][D] dequantized latents of the valid selected entries
    rope_sel: float64 [S][R] or None
    returns (out float64 [H][D], lse float64 [H])
    """
    q = bf16_bits_to_f64(q_bits)
    H = q.shape[0]
    D = c_sel.shape[1] if c_sel.ndim == 2 else q.shape[1]
    if c_sel.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    logits = q[:, :D] @ c_sel.T
    if rope_sel is not None:
        logits = logits + q[:, D:] @ rope_sel.T
    logits = sigma * logits
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ c_sel) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def valid_slots(indices, seq_len):
    """The selected positions that take part: not -1 and below the length."""
    idx = np.asarray(indices, dtype=np.int64)
    return idx[(idx >= 0) & (idx < seq_len)]


def merge_partials(out_a, lse_a, out_b, lse_b):
    """Combine two attention results over disjoint entry sets via their lse."""
    m = np.maximum(lse_a, lse_b)
    wa = np.where(np.isfinite(lse_a), np.exp(lse_a - m), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(lse_b - m), 0.0)
    out = (wa[:, None] * out_a + wb[:, None] * out_b) / (wa + wb)[:, None]
    return out, m + np.log(wa + wb)
