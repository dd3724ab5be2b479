"""Paged-cache addressing and bytes-per-token arithmetic of the oracle.

Sources:
  [P1] section "why the KV cache became the bottleneck": the global KV stays
       resident in HBM and dominates runtime KV use at long lengths; the
       per-token global KV shrank from 389,120 B (V1) to 48,068 B (V3.2),
       3,514 B (V4-Flash) and 890 B (V4.1-Flash).
  [P1] introduction: 890 B is about a quarter of V4-Flash and about 1/437 of V1.
  [P1] section "FP4 KV cache": one E4M3 scale per 16 E2M1 channels.

Readings (the pages give no cache layout):
  * The cache is paged in blocks of 64 token slots; position p of sequence b
    lives in physical row block_table[b][p // 64] * 64 + p % 64.
  * Appending a token writes position seq_len (the old length); the token is
    visible to the same step's selection and attention.
  * A packed 512-channel latent takes 256 + 32 = 288 bytes.  How the pages'
    890 B splits across entries is not given; 890 = 2.5 x 356 is one reading
    (parity unpinned: nothing on the pages fixes it) and no kernel uses it.
"""

import numpy as np

PAGE_TOKENS = 64

# Global-KV bytes per token per model generation ([P1] bottleneck section).
BYTES_PER_TOKEN_HISTORY = {
    "DeepSeek-V1": 389_120,
    "DeepSeek-V3.2": 48_068,
    "DeepSeek-V4-Flash": 3_514,
    "DeepSeek-V4.1-Flash": 890,
}


def physical_row(block_table, b, p, page_tokens=PAGE_TOKENS):
    """Physical cache row of logical position p of sequence b."""
    return int(block_table[b][p // page_tokens]) * page_tokens + p % page_tokens


def physical_rows(block_table_row, positions, page_tokens=PAGE_TOKENS):
    """Vectorised physical_row for one sequence."""
    pos = np.asarray(positions, dtype=np.int64)
    bt = np.asarray(block_table_row, dtype=np.int64)
    return bt[pos // page_tokens] * page_tokens + pos % page_tokens


def fp4_bytes_per_token(latent_dim=512, group=16):
    """Bytes of one FP4 latent: one nibble per channel plus one scale per group."""
    return latent_dim // 2 + latent_dim // group


def entry_bytes(latent_dim=512, rope_dim=0, idx_dim=0, idx_bytes=0):
    """Bytes one cached token occupies in this library's layout."""
    return fp4_bytes_per_token(latent_dim) + 2 * rope_dim + idx_dim * idx_bytes
