"""Seeded synthetic inputs for the five decode / prefill workloads.

This module only draws random numbers and arranges them in the shapes of the
workloads; it holds none of the method's arithmetic (no packing, scoring,
selection or attention).  Both the GPU tests and the CPU oracle read the same
arrays from here.

Every tensor comes from its own PCG64 stream, spawned in a fixed, named order
from SeedSequence(1000 + workload id), so a tensor does not change when
another one is added or resized.  Per-(layer, sequence) latents get their own
child stream so one sequence can be regenerated without the others.

Value laws (all workloads): N(0, 1); the KV latent additionally has 1 % of its
channels (floor(0.01 * 512) = 5, drawn once per KV layer) multiplied by 20.
bf16 tensors are drawn in float32 and rounded to nearest-even bf16; they are
returned as uint16 bit patterns.
"""

from dataclasses import dataclass, field
import math

import numpy as np

LATENT = 512
IDX_DIM = 64
IDX4_DIM = 128   # multi-head indexer: key / query-head width
IDX4_HEADS = 32  # multi-head indexer: query heads
PAGE = 64


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    heads: int
    top_k: int
    sigma: float
    seq_lens: tuple = ()
    rope_dim: int = 0
    idx_dtype: str = "bf16"
    permuted_tables: bool = False
    hierarchical: bool = False
    pool_blocks: int = 2048
    pool_block_tokens: int = 8
    layers: int = 1            # attention layers per step
    reindex_layers: int = 0    # of which re-score the pool (after one Full layer)
    reuse_layers: int = 0      # of which reuse the Full layer's indices
    kv_pools: int = 1          # distinct KV pools (one per layer when Reuse keeps own KV)
    append: bool = False
    extra: dict = field(default_factory=dict)


def _loguniform_lens(n, lo, hi, seed_seq):
    g = np.random.Generator(np.random.PCG64(seed_seq))
    return tuple(int(round(math.exp(v))) for v in g.uniform(math.log(lo), math.log(hi), size=n))


def workload(wid):
    """The workloads (tiny plumbing, 8 x 64K decode, CED prefill, 1M hierarchical, mixed serving, the 1M
    hierarchical case with the multi-head FP4 indexer, the 20-layer decoder schedule at top-K 512, CED at
    hidden 5120)."""
    if wid == 1:
        return Workload(1, "tiny_b1_4k", batch=1, heads=16, top_k=256, sigma=1 / math.sqrt(512),
                        seq_lens=(4096,), idx_dtype="f32")
    if wid == 2:
        return Workload(2, "decode_b8_64k_rope", batch=8, heads=64, top_k=2048, sigma=1 / math.sqrt(576),
                        seq_lens=(65536,) * 8, rope_dim=64, idx_dtype="bf16", permuted_tables=True)
    if wid == 3:
        return Workload(3, "ced_prefill_16k_x20", batch=0, heads=0, top_k=0, sigma=0.0,
                        extra=dict(tokens=16384, hidden=4096, layers=20, kv=512, z=64))
    if wid == 4:
        return Workload(4, "decode_1m_hierarchical", batch=1, heads=64, top_k=2048, sigma=1 / math.sqrt(512),
                        seq_lens=(1 << 20,), idx_dtype="bf16", hierarchical=True, layers=4, reindex_layers=3)
    if wid == 5:
        ss = np.random.SeedSequence(1000 + 5).spawn(1)[0]
        lens = _loguniform_lens(32, 4096, 262144, ss)
        return Workload(5, "mixed_serving_32_reuse4", batch=32, heads=64, top_k=2048, sigma=1 / math.sqrt(512),
                        seq_lens=lens, idx_dtype="bf16", permuted_tables=True, layers=4, reuse_layers=3,
                        kv_pools=4, append=True)
    if wid == 6:
        # the 1M-token case with the multi-head indexer: FP4 keys of 128 dims, 32 query heads
        return Workload(6, "decode_1m_fp4_indexer", batch=1, heads=64, top_k=2048, sigma=1 / math.sqrt(512),
                        seq_lens=(1 << 20,), idx_dtype="fp4", hierarchical=True, layers=4, reindex_layers=3,
                        extra=dict(idx_heads=IDX4_HEADS))
    if wid == 7:
        # the decoder's own shapes: top-K 512, 20 layers over one KV source in 5 groups of 4 (the first group
        # Full + 3 Reuse, the others Reindex + 3 Reuse), multi-head FP4 indexer; raw latents are finished
        # (RMSNorm, RoPE, pack) with the indexer key projected from the cached entry
        return Workload(7, "decode_1m_decoder_x20", batch=1, heads=64, top_k=512, sigma=1 / math.sqrt(512),
                        seq_lens=(1 << 20,), idx_dtype="fp4", hierarchical=True, layers=20, reindex_layers=4,
                        reuse_layers=15, extra=dict(idx_heads=IDX4_HEADS, group_size=4, finish=True))
    if wid == 10:
        # the 20-layer decoder schedule with each layer's sliding-window branch (FP8 window of 128, merged with
        # the global branch)
        return Workload(10, "decode_1m_decoder_x20_swa", batch=1, heads=64, top_k=512, sigma=1 / math.sqrt(512),
                        seq_lens=(1 << 20,), idx_dtype="fp4", hierarchical=True, layers=20, reindex_layers=4,
                        reuse_layers=15, extra=dict(idx_heads=IDX4_HEADS, group_size=4, finish=True, swa=True))
    if wid == 8:
        # CED projection at the model's hidden size 5120
        return Workload(8, "ced_prefill_16k_x20_h5120", batch=0, heads=0, top_k=0, sigma=0.0,
                        extra=dict(tokens=16384, hidden=5120, layers=20, kv=512, z=64))
    if wid == 9:
        # CED projection followed by the finish (RMSNorm, RoPE, pack) and the FP4 indexer key from the entry
        return Workload(9, "ced_prefill_16k_x20_finished", batch=0, heads=0, top_k=0, sigma=0.0,
                        extra=dict(tokens=16384, hidden=4096, layers=20, kv=512, z=0, finish=True))
    raise ValueError(wid)


# Stream names, in spawn order.  Appending new names at the end keeps old streams stable.
_NAMES = ("lens", "latent", "outliers", "idx_keys", "q_idx", "q", "rope", "tables", "append", "ced_h",
          "ced_wkv", "ced_wz", "misc", "idx_keys4", "q_idx4", "w_idx", "gamma", "w_idx_kv")


class Streams:
    """Named PCG64 generators for one workload id (or any integer seed)."""

    def __init__(self, wid, salt=0):
        root = np.random.SeedSequence(1000 + wid + 7919 * salt)
        self._children = dict(zip(_NAMES, root.spawn(len(_NAMES))))

    def gen(self, name, *sub):
        ss = self._children[name]
        for s in sub:  # deterministic sub-stream: spawn_key extension
            ss = np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + (int(s),))
        return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (input storage format only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def outlier_channels(st, layer, dim=LATENT, frac=0.01):
    g = st.gen("outliers", layer)
    return np.sort(g.choice(dim, size=int(math.floor(frac * dim)), replace=False))


def latent_rows(st, layer, seq, n, dim=LATENT, outlier_gain=20.0):
    """fp32 [n][dim] KV latent of (layer, sequence): N(0,1), outlier channels x20."""
    g = st.gen("latent", layer, seq)
    x = g.standard_normal((n, dim), dtype=np.float32)
    x[:, outlier_channels(st, layer, dim)] *= np.float32(outlier_gain)
    return x


def idx_keys(st, seq, n, dtype, dim=IDX_DIM):
    """Indexer keys of one sequence: fp32 array, or bf16 bits (uint16)."""
    x = st.gen("idx_keys", seq).standard_normal((n, dim), dtype=np.float32)
    return x if dtype == "f32" else to_bf16_bits(x)


def idx4_keys(st, seq, n, dim=IDX4_DIM):
    """fp32 [n][128] multi-head indexer keys before they are stored as FP4: N(0, 1)."""
    return st.gen("idx_keys4", seq).standard_normal((n, dim), dtype=np.float32)


def q_idx_heads(st, layer, batch, heads=IDX4_HEADS, dim=IDX4_DIM):
    """fp16 [batch][heads][128] indexer query heads: N(0, 1) rounded to fp16."""
    return st.gen("q_idx4", layer).standard_normal((batch, heads, dim), dtype=np.float32).astype(np.float16)


def w_idx(st, layer, batch, heads=IDX4_HEADS):
    """fp32 [batch][heads] per-head indexer weights: N(0, 1 / heads)."""
    return st.gen("w_idx", layer).standard_normal((batch, heads), dtype=np.float32) / np.float32(math.sqrt(heads))


def kv_finish_inputs(st, layers, key_dim=IDX4_DIM):
    """RMSNorm weights fp32 [layers][512] ~ U(0.25, 1) and the indexer-key projection from the main KV,
    bf16 bits [layers][128][512] ~ N(0, 1/512) (out x in)."""
    gamma = st.gen("gamma").uniform(0.25, 1.0, size=(layers, LATENT)).astype(np.float32)
    w = st.gen("w_idx_kv").standard_normal((layers, key_dim, LATENT), dtype=np.float32) / np.float32(math.sqrt(LATENT))
    return gamma, to_bf16_bits(w)


def rope_rows(st, layer, seq, n, dim):
    return to_bf16_bits(st.gen("rope", layer, seq).standard_normal((n, dim), dtype=np.float32))


def q_idx(st, layer, batch, dim=IDX_DIM):
    return st.gen("q_idx", layer).standard_normal((batch, dim), dtype=np.float32)


def q_heads(st, layer, batch, heads, width):
    return to_bf16_bits(st.gen("q", layer).standard_normal((batch, heads, width), dtype=np.float32))


def block_tables(st, seq_lens, permuted, extra_blocks=0, page=PAGE):
    """Block tables [B][max_blocks] over one shared pool.

    Each sequence owns ceil(len / 64) (+ extra_blocks) physical blocks; the
    pool is the concatenation of all of them, randomly permuted when asked.
    returns (tables int32 [B][maxb], num_blocks)
    """
    need = [-(-n // page) + extra_blocks for n in seq_lens]
    total = int(sum(need))
    ids = np.arange(total, dtype=np.int32)
    if permuted:
        ids = st.gen("tables").permutation(total).astype(np.int32)
    maxb = max(need) if need else 0
    tables = np.full((len(seq_lens), maxb), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(need):
        tables[b, :k] = ids[off : off + k]
        off += k
    return tables, total


def ced_inputs(st, tokens, hidden, layers, kv=LATENT, z=IDX_DIM, w_std=0.02):
    """H bf16 [T][hidden] ~ N(0,1); W_kv bf16 [L][kv][hidden], W_z bf16 [L][z][hidden] ~ N(0, 0.02^2).

    Weights are generated in the out x in orientation the library consumes.
    """
    h = to_bf16_bits(st.gen("ced_h").standard_normal((tokens, hidden), dtype=np.float32))
    wkv = to_bf16_bits(st.gen("ced_wkv").standard_normal((layers, kv, hidden), dtype=np.float32) * np.float32(w_std))
    wz = to_bf16_bits(st.gen("ced_wz").standard_normal((layers, z, hidden), dtype=np.float32) * np.float32(w_std))
    return h, wkv, wz
