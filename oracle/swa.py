"""The sliding-window (SWA) branch of the oracle: FP8 window entries and their merge with the global branch.

Sources:
  [P1] section "KV bottleneck": DeepSeek-V4 runs a global attention branch
       over the whole context (main KV + indexer K) next to a local
       sliding-window branch whose state is bounded by the fixed window.
  [P1] section "Causal Encoder-Decoder": V4.1-Flash's window n_win is 128;
       each layer's local keys and values come from its own hidden state.
  [P1] section "FP4 KV cache": the quantization-sensitive SWA KV stays in FP8.
  [P4] section 2: the first encoder layers are pure SWA with window 128.

Readings taken where the pages are silent (each is listed in the design notes):
  * A window entry is the layer's 512-channel local latent of one token, used
    as both key and value like the global entries; it has no rope part (the
    query's rope dims, if any, do not enter SWA logits).
  * FP8 is E4M3FN (the variant whose 448 maximum the FP4 scales already use)
    with one fp32 scale per token: s = fl32(amax / 448), element code =
    E4M3_RNE(fl32(x / s)) with the sign of x, saturating at 448; amax == 0
    gives s = 0 and zero codes.
  * The window of a sequence of n positions (the current token included) is
    positions max(0, n - 128) .. n - 1, kept in a ring of 128 slots
    (slot = position mod 128).
  * The two branches are merged as one softmax over the union of the selected
    global entries and the window entries (the same query and softmax scale):
    the lse-weighted merge of the two branch results.

Parity pins (tests/test_oracle_swa.py): the FP8 encoder against the
exhaustive E4M3 table (every code's value round-trips), the half-ulp error
bound of the pack, the window's slots for short and long sequences, and the
merge against attention computed directly over the concatenated entries.
"""

import numpy as np

from . import attention, fp4

WINDOW = 128
E4M3_MAX = 448.0


def swa_pack(x):
    """x float32 [n][C] -> (codes uint8 [n][C] E4M3FN, scales float32 [n])."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("swa_pack expects float32 input")
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    q = (x / safe[..., None]).astype(np.float32)  # fp32 quotient
    mag = fp4.e4m3_encode(np.abs(q).astype(np.float64)).astype(np.int64)
    sign = np.signbit(x).astype(np.int64) << 7
    codes = np.where((s > 0)[..., None], mag | sign, 0).astype(np.uint8)
    return codes, s


def swa_unpack(codes, scales):
    """(codes, scales) -> float64 [n][C] = E4M3 value * scale."""
    return fp4.e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def window_positions(n, window=WINDOW):
    """Positions of the window of a sequence of n positions (current token included)."""
    return np.arange(max(0, n - window), n, dtype=np.int64)


def window_slot(positions, window=WINDOW):
    return np.asarray(positions, dtype=np.int64) % window


def swa_attention(q_bits, win_entries, sigma, latent_dim=512):
    """Attention of every head over the window entries (float64 [w][512]); the query's rope dims are unused."""
    q = np.asarray(q_bits)[:, :latent_dim]
    return attention.sparse_attention(q, win_entries, sigma)


def merge(out_g, lse_g, out_s, lse_s):
    """One softmax over both branches' entries, from the two branch results (lse-weighted).

    Heads with neither branch holding an entry keep o = 0 and lse = -inf."""
    lse_g, lse_s = np.asarray(lse_g, dtype=np.float64), np.asarray(lse_s, dtype=np.float64)
    both = ~np.isfinite(lse_g) & ~np.isfinite(lse_s)
    with np.errstate(invalid="ignore", divide="ignore"):
        out, lse = attention.merge_partials(out_g, np.where(both, 0.0, lse_g), out_s, lse_s)
    out[both] = 0.0
    lse[both] = -np.inf
    return out, lse
