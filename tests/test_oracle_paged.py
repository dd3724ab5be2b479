"""Pins of the oracle's bytes-per-token arithmetic and paged addressing.

- 512 FP4 channels take 256 + 32 = 288 bytes;
- the pages' bytes-per-token history and the ratios they state
  (about 1/4 of V4-Flash, about 1/437 of V1);
- physical rows for hand-worked block tables.
"""

import numpy as np

from oracle import paged


def test_fp4_bytes_per_token():
    assert paged.fp4_bytes_per_token(512) == 288
    assert paged.entry_bytes(512, rope_dim=64) == 288 + 128
    assert paged.entry_bytes(512, idx_dim=64, idx_bytes=2) == 288 + 128


def test_history_and_ratios(golden):
    g = golden("kv_facts.json")
    hist = g["bytes_per_token_history"]["value"]
    assert hist == paged.BYTES_PER_TOKEN_HISTORY
    r4 = hist["DeepSeek-V4.1-Flash"] / hist["DeepSeek-V4-Flash"]
    assert abs(r4 - g["ratio_vs_v4_flash"]["value"]) <= g["ratio_vs_v4_flash"]["tolerance"]
    r1 = hist["DeepSeek-V1"] / hist["DeepSeek-V4.1-Flash"]
    assert abs(r1 - g["ratio_vs_v1"]["value"]) <= g["ratio_vs_v1"]["tolerance"]
    # an FP4 latent alone is well under the model's whole 890 B/token budget
    assert paged.fp4_bytes_per_token(512) < hist["DeepSeek-V4.1-Flash"]


def test_physical_rows_by_hand():
    table = np.array([[5, 2, 9], [0, 1, -1]])
    assert paged.physical_row(table, 0, 0) == 320
    assert paged.physical_row(table, 0, 63) == 383
    assert paged.physical_row(table, 0, 64) == 128
    assert paged.physical_row(table, 0, 130) == 9 * 64 + 2
    assert paged.physical_row(table, 1, 70) == 70
    assert paged.physical_rows(table[0], [0, 64, 130]).tolist() == [320, 128, 578]
