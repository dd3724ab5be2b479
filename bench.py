#!/usr/bin/env python3
"""Benchmark of the sparse FP4-KV decode path on one MI355X.

Default workload (the 1M-token case): one sequence of 1,048,576 cached tokens,
FP4 latent (512 ch), bf16 indexer keys, 64 heads, top-K 2048; a step appends
the new token's KV (pack) and runs one Full layer (scan of every key, block
maxima, 2048 x 8 candidate pool, its own top-K) plus three Reindex layers
(re-score the pool, own top-K), each followed by sparse FP4 decode attention.

Other workloads (--workload): decode_b8_64k_rope (8 x 65,536 tokens, rope
side-band, permuted page tables, one Full layer), mixed_serving_32_reuse4 (32
requests with log-uniform lengths, append to 4 KV layers, one Full selection
reused by 4 attentions), ced_prefill_16k_x20 (CED projection GEMM with the
fused pack; ced_prefill_16k_x20_h5120 at hidden 5120;
ced_prefill_16k_x20_finished with RMSNorm, RoPE and the FP4 indexer key from
the cached entry), tiny_b1_4k,
decode_1m_fp4_indexer (the 1M case with FP4 indexer keys of 128 dims scored by
32 weighted query heads), decode_1m_decoder_x20 (the decoder's 20-layer
Full / Reindex / Reuse schedule at top-K 512 over one KV source; _swa adds
each layer's FP8 sliding-window branch merged with the global one).

Timing: inputs are resident in HBM; R replicas of the cache rotate so every
step reads data evicted from the 256 MB last-level cache; each replica's step
is captured once as a HIP graph and replayed; W untimed steps, then exactly K
timed steps between two synchronizations.  The dominant kernel is timed
separately with HIP events around each of its launches (eager steps on the
same stream).  The CPU oracle is timed afterwards on the host for a bounded
sample of the same workload.

Prints one JSON line on stdout.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FINISH_EPS, FINISH_THETA = 1e-6, 10000.0  # RMSNorm epsilon and RoPE base of the finishing workloads
METRIC = "sparse FP4-KV decode attn queries/s + achieved HBM GB/s vs MI355X peak"
WORKLOADS = ("decode_1m_hierarchical", "decode_b8_64k_rope", "mixed_serving_32_reuse4", "ced_prefill_16k_x20",
             "tiny_b1_4k", "decode_1m_fp4_indexer", "decode_1m_decoder_x20", "ced_prefill_16k_x20_h5120",
             "ced_prefill_16k_x20_finished", "decode_1m_decoder_x20_swa")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"index_scan": "indexer.hip", "pool_score": "indexer.hip", "sparse_attn": "attention.hip",
                  "ced_project": "ced.hip"}


def kernel_source_sha(kernel):
    import hashlib

    path = os.path.join(ROOT, "sparse_attention_fp4_kv_amd", "csrc", KERNEL_SOURCES[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def usable_cores():
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()
        if quota != "max":
            n = min(n, max(1, int(int(quota) // int(period))))
    except Exception:
        pass
    return n


# --------------------------------------------------------------------------- decode workloads
class Decode:
    """Shared machinery of the decode workloads (select + attention per layer)."""

    def __init__(self, w, replicas, dev):
        import torch

        from sparse_attention_fp4_kv_amd import csa2, workloads as wl

        self.torch, self.csa2, self.wl = torch, csa2, wl
        self.w, self.dev = w, dev
        self.st = wl.Streams(w.wid)
        self.replicas = replicas

    # pack host latents of sequence b into the physical rows of `layer`
    def _fill(self, layer, table_row, n, latent=None, keys=None, rope=None, chunk=1 << 17):
        torch, csa2 = self.torch, self.csa2
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            pos = np.arange(s, e)
            rows = torch.from_numpy(table_row[pos // 64].astype(np.int64) * 64 + pos % 64).to(self.dev)
            if latent is not None:
                c, sc = csa2.csa2_fp4_pack(torch.from_numpy(latent[s:e]).to(self.dev))
                layer.codes[rows] = c
                layer.scales[rows] = sc
            if keys is not None and layer.idx_dtype == "fp4":
                c, sc = csa2.csa2_fp4_pack(torch.from_numpy(keys[s:e]).to(self.dev))
                layer.idx_keys[rows] = c
                layer.idx_scales[rows] = sc
            elif keys is not None:
                k = keys[s:e] if keys.dtype == np.float32 else keys[s:e].view(np.int16)
                layer.idx_keys[rows] = torch.from_numpy(np.ascontiguousarray(k)).to(self.dev)
            if rope is not None:
                layer.rope[rows] = torch.from_numpy(rope[s:e].view(np.int16)).to(self.dev)

    def clone_layer(self, layer):
        c = self.csa2.PagedLayer.__new__(self.csa2.PagedLayer)
        c.__dict__.update(layer.__dict__)
        for k in ("codes", "scales", "rope", "idx_keys", "idx_scales"):
            t = getattr(layer, k)
            setattr(c, k, t.clone() if t is not None else None)
        return c


class Decode1M(Decode):
    """1M-token hierarchical decode: Full + 3 Reindex layers over one shared KV and key pool.

    Indexer keys are bf16[64] with one fp32 query, or (idx_dtype "fp4") FP4[128]
    scored by 32 fp16 query heads with fp32 weights."""

    def __init__(self, w, replicas, dev, cpu_needed):
        super().__init__(w, replicas, dev)
        torch, csa2, wl = self.torch, self.csa2, self.wl
        n = w.seq_lens[0]
        self.n, self.H, self.K, self.P, self.L = n, w.heads, w.top_k, w.pool_blocks, w.layers
        self.fp4 = w.idx_dtype == "fp4"
        self.IH = w.extra.get("idx_heads", 1)
        self.finish = w.extra.get("finish", False)  # raw latents finished (norm, RoPE, pack, key) on the way in
        t0 = time.time()
        self.latent = wl.latent_rows(self.st, 0, 0, n)
        if self.finish:
            self.gamma, self.w_kv_idx = wl.kv_finish_inputs(self.st, 1)
            self.gamma_d = torch.from_numpy(self.gamma[0].copy()).to(dev)
            self.w_kv_idx_d = torch.from_numpy(self.w_kv_idx[0].view(np.int16).copy()).to(dev)
        if self.fp4:
            self.keys = wl.idx4_keys(self.st, 0, n)
            self.q_idx = [wl.q_idx_heads(self.st, l, 1, self.IH) for l in range(self.L)]
            self.w_idx = [wl.w_idx(self.st, l, 1, self.IH) for l in range(self.L)]
        else:
            self.keys = wl.idx_keys(self.st, 0, n, "bf16")
            self.q_idx = [wl.q_idx(self.st, l, 1) for l in range(self.L)]
            self.w_idx = [None] * self.L
        self.q = [wl.q_heads(self.st, l, 1, self.H, 512) for l in range(self.L)]
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        nb = n // 64
        table = np.arange(nb, dtype=np.int32)
        base = csa2.PagedLayer(nb, idx_dtype=w.idx_dtype, idx_heads=self.IH, device=dev)
        if self.finish:
            self._fill_finished(base, n)
        else:
            self._fill(base, table, n, latent=self.latent, keys=self.keys)
        self.layers = [base] + [self.clone_layer(base) for _ in range(replicas - 1)]
        bt = torch.from_numpy(table[None].copy()).to(dev)
        self.batch = csa2.Batch(bt, torch.tensor([n], dtype=torch.int32, device=dev), n)
        self.batch_prev = csa2.Batch(bt, torch.tensor([n - 1], dtype=torch.int32, device=dev), n)
        self.new_latent = torch.from_numpy(self.latent[n - 1 : n].copy()).to(dev)
        nk = self.keys[n - 1 : n]
        self.new_key = torch.from_numpy((nk if self.fp4 else nk.view(np.int16)).copy()).to(dev)
        self.q_idx_d = [torch.from_numpy(q).to(dev) for q in self.q_idx]
        self.w_idx_d = [torch.from_numpy(x).to(dev) if x is not None else None for x in self.w_idx]
        self.q_d = [torch.from_numpy(q.view(np.int16)).to(dev) for q in self.q]
        self.sel_ws = csa2.workspace(csa2.index_select_workspace_bytes(1, n, self.K, self.P), dev)
        self.lead_layers = list(range(self.L))  # every layer selects (Full, then Reindex)
        self.idx = torch.empty((self.L, 1, self.K), dtype=torch.int32, device=dev)
        self.pool = torch.empty((1, self.P), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.L, 1, self.H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.L, 1, self.H), dtype=torch.float32, device=dev)
        self.kf64 = None
        self.o_entries = None
        if cpu_needed and self.finish:
            import oracle
            parts = [oracle.latent.kv_entry(self.latent[s:s + (1 << 17)], np.arange(s, min(n, s + (1 << 17))),
                                            self.gamma[0], FINISH_EPS, FINISH_THETA, self.w_kv_idx[0])
                     for s in range(0, n, 1 << 17)]
            self.o_entries = (np.concatenate([p[1] for p in parts]), np.concatenate([p[2] for p in parts]))
            self.kf64 = oracle.indexer.fp4_keys_to_f64(np.concatenate([p[4] for p in parts]),
                                                       np.concatenate([p[5] for p in parts]))
            del parts
        elif cpu_needed:
            import oracle
            if self.fp4:
                self.kf64 = oracle.indexer.fp4_keys_to_f64(*oracle.fp4.fp4_pack(self.keys))
            else:
                self.kf64 = oracle.indexer.keys_to_f64(self.keys, "bf16")
        if type(self) is Decode1M:
            self._workspaces()
        torch.cuda.synchronize()

    queries_per_step = property(lambda self: self.L)
    dominant = "index_scan"

    def _workspaces(self):
        """Reindex and multi-layer attention workspaces (after the subclass has fixed its layer plan)."""
        csa2, dev = self.csa2, self.dev
        nre = max(1, len(self.lead_layers) - 1)
        self.reidx_ws = csa2.workspace(csa2.reindex_layers_workspace_bytes(nre, 1, self.K, self.P), dev)
        self.attn_ws = csa2.workspace(csa2.attn_layers_workspace_bytes(self.L, 1, self.H, self.K,
                                                                       getattr(self, "swa", False)), dev)

    def _select(self, layer, idx_of_lead):
        """Full selection with the pool (the new token's row appended in the scan's launch, or by the
        finishing append before it), then every Reindex layer over that pool in two launches."""
        csa2 = self.csa2
        l0 = self.lead_layers[0]
        if self.finish:
            self._append(layer)
            csa2.csa2_index_select(layer, self.batch, self.q_idx_d[l0], self.K, csa2.FULL, pool_blocks=self.P,
                                   want_pool=True, ws=self.sel_ws, indices=idx_of_lead[0], pool_out=self.pool,
                                   w_idx=self.w_idx_d[l0])
        else:
            csa2.csa2_index_select_append(layer, self.batch, self.q_idx_d[l0], self.K,
                                          [(layer, self.new_latent, None, self.new_key)], pool_blocks=self.P,
                                          want_pool=True, ws=self.sel_ws, indices=idx_of_lead[0], pool_out=self.pool,
                                          w_idx=self.w_idx_d[l0])
        rest = self.lead_layers[1:]
        if rest:
            csa2.csa2_index_reindex_layers(layer, self.batch, [(self.q_idx_d[l], self.w_idx_d[l]) for l in rest],
                                           self.K, self.pool, self.P, ws=self.reidx_ws, indices=idx_of_lead[1:])

    def _fill_finished(self, layer, n, chunk=1 << 17):
        """Identity page table: finish raw latents of positions [s, e) straight into rows [s, e)."""
        torch, csa2 = self.torch, self.csa2
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            c = torch.from_numpy(self.latent[s:e][None].copy()).to(self.dev)
            codes, scales, kc, ks, _, _ = csa2.csa2_kv_finish_rows(c, self.gamma_d[None], FINISH_EPS, FINISH_THETA,
                                                                   self.w_kv_idx_d[None], pos0=s)
            layer.codes[s:e], layer.scales[s:e] = codes[0], scales[0]
            layer.idx_keys[s:e], layer.idx_scales[s:e] = kc[0], ks[0]

    def _append(self, layer):
        if self.finish:
            self.csa2.csa2_kv_append_finished(layer, self.batch_prev, self.new_latent, self.gamma_d, FINISH_EPS,
                                              FINISH_THETA, self.w_kv_idx_d)
        else:
            self.csa2.csa2_kv_append(layer, self.batch_prev, self.new_latent, idx_key=self.new_key)

    def _oracle_kv(self, v):
        """Oracle float64 cache entries of positions v."""
        import oracle

        if self.o_entries is not None:
            return oracle.fp4.fp4_unpack(self.o_entries[0][v], self.o_entries[1][v])
        return oracle.fp4.fp4_unpack(*oracle.fp4.fp4_pack(self.latent[v]))

    def step_sequential(self, r):
        """The same step as one call per layer and kind, as a decoder that runs other work between its layers
        would issue it: append, then per layer its selection (Full with the pool, or Reindex) and its
        attention, each its own launches."""
        csa2, layer = self.csa2, self.layers[r]
        csa2.csa2_kv_append(layer, self.batch_prev, self.new_latent, idx_key=self.new_key)
        for l in range(self.L):
            if l == 0:
                csa2.csa2_index_select(layer, self.batch, self.q_idx_d[0], self.K, csa2.FULL, pool_blocks=self.P,
                                       want_pool=True, ws=self.sel_ws, indices=self.idx[0], pool_out=self.pool,
                                       w_idx=self.w_idx_d[0])
            else:
                csa2.csa2_index_select(layer, self.batch, self.q_idx_d[l], self.K, csa2.REINDEX, pool_in=self.pool,
                                       pool_blocks=self.P, ws=self.sel_ws, indices=self.idx[l], w_idx=self.w_idx_d[l])
            csa2.csa2_sparse_fp4_decode_attn(layer, self.batch, self.q_d[l], self.idx[l], self.w.sigma,
                                             ws=self.attn_ws, out=self.out[l], lse=self.lse[l])

    def step(self, r):
        """append + Full select with the pool (one scan launch, one select launch), the 3 Reindex layers
        (one pool-scoring launch, one select launch), the 4 attentions (one launch, one combine)."""
        csa2, layer = self.csa2, self.layers[r]
        self._select(layer, [self.idx[l] for l in range(self.L)])
        csa2.csa2_sparse_fp4_decode_attn_layers([(layer, self.q_d[l], self.idx[l]) for l in range(self.L)],
                                                self.batch, self.w.sigma, ws=self.attn_ws,
                                                outs=[self.out[l] for l in range(self.L)],
                                                lses=[self.lse[l] for l in range(self.L)])

    def attn_bytes(self):
        """Algorithmic bytes of the step's attention launch: every layer's gathered entries, query, indices,
        output and lse (the windows too when the layers have them)."""
        L, K, H = self.L, self.K, self.H
        win = L * 128 * (512 + 4) + L * (512 * 4) if getattr(self, "swa", False) else 0
        return L * (K * 288 + H * 512 * 2 + K * 4 + H * 512 * 4 + H * 4) + win

    # indexer key bytes per token (FP4: 64 B of codes + 8 scales) and query bytes per selection
    key_bytes = property(lambda self: 72 if self.fp4 else 128)
    qsel_bytes = property(lambda self: self.IH * 128 * 2 + self.IH * 4 if self.fp4 else 64 * 4)

    def algorithmic_bytes(self):
        n, K, P, H, L = self.n, self.K, self.P, self.H, self.L
        scan = n * self.key_bytes + self.qsel_bytes
        reindex = (L - 1) * (P * 8 * self.key_bytes + self.qsel_bytes)
        kv = L * K * 288
        qio = L * (H * 512 * 2 + H * 512 * 4 + H * 4)
        append = 512 * 4 + 288 + (128 * 4 + 72 if self.fp4 else 128 + 128)
        return scan + reindex + kv + qio + append

    def dominant_bytes(self):
        return self.n * self.key_bytes + self.qsel_bytes  # every key once + the query

    def dominant_flops(self):
        return 2 * self.n * self.IH * 128 if self.fp4 else 0  # fp16 MFMA: every key against every head

    def oracle_step(self):
        import oracle

        w = [x[0] if x is not None else None for x in self.w_idx]
        idx, pool = oracle.indexer.full_select(self.q_idx[0][0], self.kf64, self.K, pool_blocks_max=self.P, w=w[0])
        sel = [idx] + [oracle.indexer.reindex_select(self.q_idx[l][0], self.kf64, self.K, pool, w=w[l])
                       for l in range(1, self.L)]
        outs = []
        for l in range(self.L):
            v = oracle.attention.valid_slots(sel[l], self.n)
            outs.append(oracle.attention.sparse_attention(self.q[l][0], self._oracle_kv(v), self.w.sigma))
        return outs

    def config(self):
        return {"workload": self.w.name, "batch": 1, "seq_len": self.n, "heads": self.H, "top_k": self.K,
                "pool": f"{self.P}x8", "layers": "1 Full + 3 Reindex", "kv_bytes_per_token": 288,
                "idx_key": f"fp4[128] (64 B codes + 8 E4M3 scales), {self.IH} fp16 query heads" if self.fp4
                else "bf16[64]", "append_per_step": 1, "replicas": self.replicas}


class DecoderX20(Decode1M):
    """The decoder's schedule at its own shapes: 20 layers over one KV source in 5 groups of 4; the first
    group's lead layer is Full (and builds the 2048 x 8 pool), the other groups' lead layers Reindex the
    pool, and the 3 other layers of each group Reuse their lead's indices.  Top-K 512, FP4 indexer keys
    scored by 32 query heads, 64 attention heads per layer."""

    def __init__(self, w, replicas, dev, cpu_needed):
        super().__init__(w, replicas, dev, cpu_needed)
        self.G = w.extra["group_size"]
        self.leads = list(range(0, self.L, self.G))
        self.lead_layers = self.leads
        self.gidx = self.torch.empty((len(self.leads), 1, self.K), dtype=self.torch.int32, device=dev)
        self.swa = w.extra.get("swa", False)
        if self.swa:  # every layer's own window of 128 local latents (FP8), one ring per layer and replica
            csa2, torch = self.csa2, self.torch
            n = self.n
            self.win_lat = [self.wl.latent_rows(self.st, 100 + l, 0, 128) for l in range(self.L)]
            self.rings = [[csa2.SwaRing(1, dev) for _ in range(self.L)] for _ in range(replicas)]
            for l in range(self.L):
                lat_d = torch.from_numpy(self.win_lat[l]).to(dev)
                for j in range(128):
                    csa2.csa2_swa_append(self.rings[0][l], torch.tensor([n - 128 + j], dtype=torch.int32, device=dev),
                                         lat_d[j:j + 1])
                for r in range(1, replicas):
                    self.rings[r][l].codes.copy_(self.rings[0][l].codes)
                    self.rings[r][l].scales.copy_(self.rings[0][l].scales)
            self.win_new = [torch.from_numpy(self.win_lat[l][127:128].copy()).to(dev) for l in range(self.L)]
        self._workspaces()
        self.torch.cuda.synchronize()

    def step(self, r):
        """The finishing append, the Full select with the pool, the 4 Reindex leads (two launches), then all
        20 layers' attention in one launch (each lead's Reuse layers take its indices; with windows, every
        layer's new window entry is appended in that launch)."""
        csa2, layer = self.csa2, self.layers[r]
        self._select(layer, [self.gidx[g] for g in range(len(self.leads))])
        jobs = []
        for g, l0 in enumerate(self.leads):
            for l in range(l0, l0 + self.G):  # the lead and its Reuse layers
                if self.swa:
                    jobs.append((layer, self.q_d[l], self.gidx[g], self.rings[r][l], self.win_new[l]))
                else:
                    jobs.append((layer, self.q_d[l], self.gidx[g]))
        csa2.csa2_sparse_fp4_decode_attn_layers(jobs, self.batch, self.w.sigma, ws=self.attn_ws,
                                                outs=[self.out[l] for l in range(self.L)],
                                                lses=[self.lse[l] for l in range(self.L)])

    def algorithmic_bytes(self):
        n, K, P, H, L = self.n, self.K, self.P, self.H, self.L
        scan = n * self.key_bytes + self.qsel_bytes
        reindex = (len(self.leads) - 1) * (P * 8 * self.key_bytes + self.qsel_bytes)
        kv = L * K * 288
        qio = L * (H * 512 * 2 + H * 512 * 4 + H * 4)
        append = 512 * 4 + 288 + 72 + (512 * 4 + 128 * 512 * 2 if self.finish else 128 * 4)
        if self.swa:  # per layer: the new window entry, and the window read once
            append += L * (512 * 4 + 512 + 4)
            kv += L * 128 * (512 + 4)
        return scan + reindex + kv + qio + append

    def oracle_step(self):
        import oracle

        w = [x[0] for x in self.w_idx]
        idx, pool = oracle.indexer.full_select(self.q_idx[0][0], self.kf64, self.K, pool_blocks_max=self.P, w=w[0])
        sel = {0: idx}
        for l0 in self.leads[1:]:
            sel[l0] = oracle.indexer.reindex_select(self.q_idx[l0][0], self.kf64, self.K, pool, w=w[l0])
        outs = []
        for l0 in self.leads:
            v = oracle.attention.valid_slots(oracle.indexer.reuse_select(sel[l0]), self.n)
            c = self._oracle_kv(v)
            for l in range(l0, l0 + self.G):
                o = oracle.attention.sparse_attention(self.q[l][0], c, self.w.sigma)
                if self.swa:
                    win = oracle.swa.swa_unpack(*oracle.swa.swa_pack(self.win_lat[l]))
                    o = oracle.swa.merge(*o, *oracle.swa.swa_attention(self.q[l][0], win, self.w.sigma))
                outs.append(o)
        return outs

    def config(self):
        c = super().config()
        c["layers"] = "20 in 5 groups of 4: Full + 3 Reuse, then 4 x (Reindex + 3 Reuse), one KV source"
        if self.swa:
            c["swa"] = ("per layer: FP8 window of 128 (E4M3 + fp32 per-token scale) in one softmax with the global "
                        "branch (the window slots run as extra splits of the attention kernel)")
        return c


class DecodeBatch(Decode):
    """Batched decode with one Full selection per step and attention (config 2 style; tiny case too)."""

    def __init__(self, w, replicas, dev, cpu_needed):
        super().__init__(w, replicas, dev)
        torch, csa2, wl = self.torch, self.csa2, self.wl
        self.B, self.H, self.K, self.R = w.batch, w.heads, w.top_k, w.rope_dim
        self.lens = list(w.seq_lens)
        tables, nb = wl.block_tables(self.st, self.lens, w.permuted_tables)
        self.tables = tables
        t0 = time.time()
        self.latents, self.keys, self.ropes = [], [], []
        base = csa2.PagedLayer(nb, rope_dim=self.R, idx_dtype=w.idx_dtype, device=dev)
        for b, n in enumerate(self.lens):
            lat = wl.latent_rows(self.st, 0, b, n)
            key = wl.idx_keys(self.st, b, n, w.idx_dtype)
            rope = wl.rope_rows(self.st, 0, b, n, self.R) if self.R else None
            self._fill(base, tables[b], n, latent=lat, keys=key, rope=rope)
            self.latents.append(lat if cpu_needed else None)
            self.keys.append(key)
            self.ropes.append(rope)
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        self.layers = [base] + [self.clone_layer(base) for _ in range(replicas - 1)]
        self.q_idx = wl.q_idx(self.st, 0, self.B)
        self.q = wl.q_heads(self.st, 0, self.B, self.H, 512 + self.R)
        self.batch = csa2.Batch(torch.from_numpy(tables).to(dev), torch.tensor(self.lens, dtype=torch.int32,
                                                                                 device=dev), max(self.lens))
        self.q_idx_d = torch.from_numpy(self.q_idx).to(dev)
        self.q_d = torch.from_numpy(self.q.view(np.int16)).to(dev)
        self.sel_ws = csa2.workspace(csa2.index_select_workspace_bytes(self.B, max(self.lens), self.K), dev)
        self.attn_ws = csa2.workspace(csa2.attn_workspace_bytes(self.B, self.H, self.K), dev)
        self.idx = torch.empty((self.B, self.K), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.B, self.H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.B, self.H), dtype=torch.float32, device=dev)
        self.kf64 = None
        if cpu_needed:
            import oracle
            self.kf64 = [oracle.indexer.keys_to_f64(k, w.idx_dtype) for k in self.keys]
        torch.cuda.synchronize()

    queries_per_step = property(lambda self: self.B)
    dominant = "index_scan"

    def step(self, r):
        csa2, layer = self.csa2, self.layers[r]
        csa2.csa2_index_select(layer, self.batch, self.q_idx_d, self.K, csa2.FULL, ws=self.sel_ws, indices=self.idx)
        csa2.csa2_sparse_fp4_decode_attn(layer, self.batch, self.q_d, self.idx, self.w.sigma, ws=self.attn_ws,
                                         out=self.out, lse=self.lse)

    def key_bytes(self):
        return 256 if self.w.idx_dtype == "f32" else 128

    def algorithmic_bytes(self):
        entry = 288 + 2 * self.R
        per = sum(n * self.key_bytes() + min(n, self.K) * entry for n in self.lens)
        qio = self.B * (self.H * (512 + self.R) * 2 + self.H * 512 * 4 + self.H * 4 + 64 * 4)
        return per + qio

    def dominant_bytes(self):
        return sum(n * self.key_bytes() for n in self.lens) + self.B * 64 * 4

    def attn_bytes(self):
        entry = 288 + 2 * self.R
        return sum(min(n, self.K) * entry for n in self.lens) + self.B * (
            self.H * (512 + self.R) * 2 + self.K * 4 + self.H * 512 * 4 + self.H * 4)

    def oracle_step(self, rows=None):
        import oracle

        outs = []
        for b in (rows if rows is not None else range(self.B)):
            n = self.lens[b]
            idx, _ = oracle.indexer.full_select(self.q_idx[b], self.kf64[b], self.K)
            v = oracle.attention.valid_slots(idx, n)
            c = oracle.fp4.fp4_unpack(*oracle.fp4.fp4_pack(self.latents[b][v]))
            rope = oracle.ced.bf16_bits_to_f64(self.ropes[b][v]) if self.R else None
            outs.append(oracle.attention.sparse_attention(self.q[b], c, self.w.sigma, rope_sel=rope))
        return outs

    def config(self):
        return {"workload": self.w.name, "batch": self.B, "seq_len": max(self.lens), "heads": self.H,
                "top_k": self.K, "rope_dim": self.R, "idx_key": f"{self.w.idx_dtype}[64]",
                "page_tables": "permuted" if self.w.permuted_tables else "identity", "replicas": self.replicas}


class MixedServing(Decode):
    """32 requests, 4 KV layers with their own pools, 1 Full selection reused by 4 attentions, append every step."""

    def __init__(self, w, replicas, dev, cpu_needed):
        super().__init__(w, replicas, dev)
        torch, csa2, wl = self.torch, self.csa2, self.wl
        self.B, self.H, self.K, self.L = w.batch, w.heads, w.top_k, w.layers
        self.lens = list(w.seq_lens)              # tokens before this step's append
        tables, nb = wl.block_tables(self.st, [n + 1 for n in self.lens], True)
        self.tables = tables
        t0 = time.time()
        self.key_pool = csa2.PagedLayer(nb, idx_dtype="bf16", device=dev)
        kv = [csa2.PagedLayer(nb, device=dev) for _ in range(self.L)]
        self.keys = []
        self.cpu_needed = cpu_needed
        for b, n in enumerate(self.lens):
            key = wl.idx_keys(self.st, b, n + 1, "bf16")
            self._fill(self.key_pool, tables[b], n, keys=key[:n])
            self.keys.append(key)
            for l in range(self.L):
                lat = wl.latent_rows(self.st, l, b, n + 1)
                self._fill(kv[l], tables[b], n, latent=lat[:n])
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        self.key_pools = [self.key_pool] + [self.clone_layer(self.key_pool) for _ in range(replicas - 1)]
        self.kv = [kv] + [[self.clone_layer(x) for x in kv] for _ in range(replicas - 1)]
        self.new_lat = [torch.from_numpy(np.stack([wl.latent_rows(self.st, l, b, n + 1)[n] for b, n in
                                                   enumerate(self.lens)])).to(dev) for l in range(self.L)]
        self.new_key = torch.from_numpy(np.stack([k[-1] for k in self.keys]).view(np.int16)).to(dev)
        bt = torch.from_numpy(tables).to(dev)
        maxn = max(self.lens) + 1
        self.batch_prev = csa2.Batch(bt, torch.tensor(self.lens, dtype=torch.int32, device=dev), maxn)
        self.batch = csa2.Batch(bt, torch.tensor([n + 1 for n in self.lens], dtype=torch.int32, device=dev), maxn)
        self.q_idx = wl.q_idx(self.st, 0, self.B)
        self.q = [wl.q_heads(self.st, l, self.B, self.H, 512) for l in range(self.L)]
        self.q_idx_d = torch.from_numpy(self.q_idx).to(dev)
        self.q_d = [torch.from_numpy(q.view(np.int16)).to(dev) for q in self.q]
        self.sel_ws = csa2.workspace(csa2.index_select_workspace_bytes(self.B, maxn, self.K), dev)
        self.attn_ws = csa2.workspace(csa2.attn_layers_workspace_bytes(self.L, self.B, self.H, self.K), dev)
        self.idx = torch.empty((self.B, self.K), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.L, self.B, self.H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.L, self.B, self.H), dtype=torch.float32, device=dev)
        self.oracle_rows = {}
        if cpu_needed:  # the CPU sample's inputs, generated here, outside its timed loop
            import oracle

            for b in range(min(self.B, self.ORACLE_SEQS)):
                n = self.lens[b] + 1
                kf = oracle.indexer.keys_to_f64(self.keys[b], "bf16")
                idx, _ = oracle.indexer.full_select(self.q_idx[b], kf, self.K)
                v = oracle.attention.valid_slots(idx, n)
                self.oracle_rows[b] = (kf, idx, [wl.latent_rows(self.st, l, b, n)[v] for l in range(self.L)])
        torch.cuda.synchronize()

    ORACLE_SEQS = 8  # sequences whose oracle inputs are prepared for the CPU baseline
    queries_per_step = property(lambda self: self.B * self.L)
    dominant = "index_scan"

    def step(self, r):
        """The new token's key (key pool) and its latent (each layer's own KV pool) appended in the scan's
        launch, one Full selection, then the 4 Reuse layers' attention over their own KV in one launch."""
        csa2 = self.csa2
        rows = [(self.key_pools[r], None, None, self.new_key)] + [(self.kv[r][l], self.new_lat[l], None, None)
                                                                  for l in range(self.L)]
        csa2.csa2_index_select_append(self.key_pools[r], self.batch, self.q_idx_d, self.K, rows, ws=self.sel_ws,
                                      indices=self.idx)
        csa2.csa2_sparse_fp4_decode_attn_layers([(self.kv[r][l], self.q_d[l], self.idx) for l in range(self.L)],
                                                self.batch, self.w.sigma, ws=self.attn_ws,
                                                outs=[self.out[l] for l in range(self.L)],
                                                lses=[self.lse[l] for l in range(self.L)])

    def algorithmic_bytes(self):
        per = sum((n + 1) * 128 for n in self.lens) + self.L * sum(min(n + 1, self.K) for n in self.lens) * 288
        qio = self.L * self.B * (self.H * 512 * 2 + self.H * 512 * 4 + self.H * 4) + self.B * 64 * 4
        append = self.L * self.B * (512 * 4 + 288) + self.B * (128 + 128)
        return per + qio + append

    def dominant_bytes(self):
        return sum((n + 1) * 128 for n in self.lens) + self.B * 64 * 4

    def attn_bytes(self):
        return self.L * (sum(min(n + 1, self.K) for n in self.lens) * 288 + self.B * (
            self.H * 512 * 2 + self.K * 4 + self.H * 512 * 4 + self.H * 4))

    def oracle_step(self, rows=None):
        """The oracle on sequences whose inputs __init__ prepared: the Full selection over every key, then
        each layer's pack of the selected latents and its attention."""
        import oracle

        outs = []
        for b in (rows if rows is not None else sorted(self.oracle_rows)):
            kf, idx0, lat_sel = self.oracle_rows[b]
            idx, _ = oracle.indexer.full_select(self.q_idx[b], kf, self.K)
            assert np.array_equal(idx, idx0)
            for l in range(self.L):
                c = oracle.fp4.fp4_unpack(*oracle.fp4.fp4_pack(lat_sel[l]))
                outs.append(oracle.attention.sparse_attention(self.q[l][b], c, self.w.sigma))
        return outs

    def config(self):
        return {"workload": self.w.name, "batch": self.B, "seq_len_max": max(self.lens) + 1,
                "seq_len_sum": sum(self.lens) + self.B, "heads": self.H, "top_k": self.K,
                "layers": "1 Full selection reused by 4 layers (own KV each)", "append_per_step": self.B * self.L,
                "replicas": self.replicas}


class CedPrefill:
    """CED projection of 16,384 tokens x hidden (4096 or 5120) into 20 layers (512 FP4 + 64 bf16 channels each)."""

    def __init__(self, w, replicas, dev, cpu_needed):
        import torch

        from sparse_attention_fp4_kv_amd import csa2, workloads as wl

        self.torch, self.csa2, self.w, self.dev = torch, csa2, w, dev
        e = w.extra
        self.T, self.Hd, self.L = e["tokens"], e["hidden"], e["layers"]
        st = wl.Streams(w.wid)
        t0 = time.time()
        self.h, self.wkv, self.wz = wl.ced_inputs(st, self.T, self.Hd, self.L)
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        self.h_d = torch.from_numpy(self.h.view(np.int16)).to(dev)
        self.wkv_d = torch.from_numpy(self.wkv.view(np.int16)).to(dev)
        self.wz_d = torch.from_numpy(self.wz.view(np.int16)).to(dev)
        self.codes = torch.empty((self.L, self.T, 256), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((self.L, self.T, 32), dtype=torch.uint8, device=dev)
        self.z = torch.empty((self.L, self.T, 64), dtype=torch.int16, device=dev)
        self.finish = e.get("finish", False)  # C finished (RMSNorm, RoPE, pack) + FP4 key from the cached entry
        if self.finish:
            self.gamma, self.w_idx = wl.kv_finish_inputs(st, self.L)
            self.gamma_d = torch.from_numpy(self.gamma).to(dev)
            self.w_idx_d = torch.from_numpy(self.w_idx.view(np.int16)).to(dev)
            self.c_ws = torch.empty((self.L, self.T, 512), dtype=torch.float32, device=dev)
            self.kc = torch.empty((self.L, self.T, 64), dtype=torch.uint8, device=dev)
            self.ks = torch.empty((self.L, self.T, 8), dtype=torch.uint8, device=dev)
            self.fin = csa2.KvFinish(gamma=self.gamma_d.data_ptr(), eps=FINISH_EPS, rope_theta=FINISH_THETA,
                                     w_idx=self.w_idx_d.data_ptr())
        self.replicas = 1
        torch.cuda.synchronize()

    queries_per_step = property(lambda self: self.T)
    dominant = "ced_project"

    def step(self, r):
        c = self.csa2
        if self.finish:
            import ctypes

            c._check(c.lib().csa2_ced_kv_project_finished(
                c._ptr(self.h_d), self.T, self.Hd, self.L, c._ptr(self.wkv_d), ctypes.byref(self.fin), 0,
                c._ptr(self.c_ws), c._ptr(self.codes), c._ptr(self.scales), c._ptr(self.kc), c._ptr(self.ks),
                c._stream()), "csa2_ced_kv_project_finished")
            return
        c._check(c.lib().csa2_ced_kv_project(c._ptr(self.h_d), self.T, self.Hd, self.L, c._ptr(self.wkv_d),
                                             c._ptr(self.wz_d), c._ptr(self.codes), c._ptr(self.scales),
                                             c._ptr(self.z), None, c._stream()), "csa2_ced_kv_project")

    def gemm_flops(self):  # the projection GEMM alone (the dominant kernel)
        return 2.0 * self.T * self.Hd * self.L * (512 if self.finish else 576)

    def flops(self):
        if self.finish:  # C (512 per layer) and the 128-dim key from the 512-dim entry
            return 2.0 * self.T * self.L * 512 * (self.Hd + 128)
        return 2.0 * self.T * self.Hd * self.L * 576

    def algorithmic_bytes(self):
        if self.finish:  # + the fp32 hand-over of C (written, read), W_idx and gamma, the FP4 key
            return (self.T * self.Hd * 2 + self.L * 512 * self.Hd * 2 + self.L * self.T * (288 + 72 + 2 * 2048)
                    + self.L * (128 * 512 * 2 + 2048))
        return self.T * self.Hd * 2 + self.L * 576 * self.Hd * 2 + self.L * self.T * (288 + 128)

    def dominant_bytes(self):
        return self.algorithmic_bytes()

    def oracle_step(self, rows=64):
        import oracle

        if self.finish:
            C, _ = oracle.ced.ced_project(self.h[:rows], self.wkv, None)
            return [oracle.latent.kv_entry(C[l], np.arange(rows), self.gamma[l], FINISH_EPS, FINISH_THETA,
                                           self.w_idx[l]) for l in range(self.L)]
        return oracle.ced.ced_project_and_pack(self.h[:rows], self.wkv, self.wz)

    def config(self):
        return {"workload": self.w.name, "tokens": self.T, "hidden": self.Hd, "layers": self.L,
                "out_per_layer": "512 FP4 (RMSNorm + RoPE) + FP4 key [128] from the entry" if self.finish
                else "512 FP4 + 64 bf16"}


def make(name, replicas, dev, cpu_needed):
    from sparse_attention_fp4_kv_amd import workloads as wl

    wid = {"tiny_b1_4k": 1, "decode_b8_64k_rope": 2, "ced_prefill_16k_x20": 3, "decode_1m_hierarchical": 4,
           "mixed_serving_32_reuse4": 5, "decode_1m_fp4_indexer": 6, "decode_1m_decoder_x20": 7,
           "ced_prefill_16k_x20_h5120": 8, "ced_prefill_16k_x20_finished": 9, "decode_1m_decoder_x20_swa": 10}[name]
    w = wl.workload(wid)
    if wid in (7, 10):
        return DecoderX20(w, replicas, dev, cpu_needed)
    if wid in (4, 6):
        return Decode1M(w, replicas, dev, cpu_needed)
    if wid == 5:
        return MixedServing(w, replicas, dev, cpu_needed)
    if wid in (3, 8, 9):
        return CedPrefill(w, replicas, dev, cpu_needed)
    return DecodeBatch(w, replicas, dev, cpu_needed)


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wk, budget_s):
    """The oracle as it stands, single-threaded and pinned to one core, on a bounded sample."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores_avail = usable_cores()
    try:
        cpu = sorted(os.sched_getaffinity(0))[0]
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {cpu})
    except Exception:
        old = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if isinstance(wk, CedPrefill):
            rows = 64
            t0 = time.time()
            reps = 0
            while reps < 1 or time.time() - t0 < budget_s:
                wk.oracle_step(rows)
                reps += 1
            dt = time.time() - t0
            fl = wk.flops() * rows * reps / wk.T
            return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                    "sample": f"{reps} x {rows}-token slices x 20 layers of the CED projection + pack (float64)",
                    "usable_cores": cores_avail, "cpu_model": cpu_model()}
        per_call_queries = None
        t0 = time.time()
        calls = 0
        queries = 0
        if isinstance(wk, Decode1M):
            while calls < 1 or time.time() - t0 < budget_s:
                wk.oracle_step()
                calls += 1
                queries += wk.L
            sample = (f"{calls} full 20-layer steps (1M-token scan, pool, 4 Reindex, 20 attentions)"
                      if isinstance(wk, DecoderX20) else
                      f"{calls} full 4-layer steps (1M-token scan, pool, 3 Reindex, 4 attentions)")
        else:
            seqs = sorted(wk.oracle_rows) if getattr(wk, "oracle_rows", None) else list(range(wk.B))
            b = 0
            while calls < 1 or time.time() - t0 < budget_s:
                wk.oracle_step(rows=[seqs[b % len(seqs)]])
                calls += 1
                queries += getattr(wk, "L", 1)
                b += 1
            sample = (f"{calls} sequences of the batch (selection + attention per sequence, float64; "
                      f"cycling over sequences {seqs[0]}..{seqs[-1]})")
        dt = time.time() - t0
        return {"value": queries / dt, "unit": "queries/s", "cores": 1, "kind": "oracle", "sample": sample,
                "seconds": round(dt, 2), "usable_cores": cores_avail, "cpu_model": cpu_model()}
    finally:
        if ctx is not None:
            ctx.unregister() if hasattr(ctx, "unregister") else None
        if old is not None:
            os.sched_setaffinity(0, old)


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m_hierarchical", choices=WORKLOADS)
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas rotated for cold reads (0: auto)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--sequential", action="store_true",
                    help="1M-token workloads: issue the step one layer at a time (separate selection and attention "
                         "calls per layer), the latency a decoder with other work between its layers would see")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size reference for "
                         "hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); sharding across GPUs (whole "
              "sequences per GPU, or one sequence's context split with one all-gather of the local top-K) is "
              "not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_fp4_kv_amd import csa2

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    csa2.lib()
    if args.calibrate_copy_mib:
        src = torch.ones(args.calibrate_copy_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    replicas = args.replicas or {"decode_1m_hierarchical": 4, "decode_b8_64k_rope": 6, "mixed_serving_32_reuse4": 3,
                                 "ced_prefill_16k_x20": 1, "tiny_b1_4k": 1, "decode_1m_fp4_indexer": 4,
                                 "decode_1m_decoder_x20": 4, "ced_prefill_16k_x20_h5120": 1,
                                 "ced_prefill_16k_x20_finished": 1, "decode_1m_decoder_x20_swa": 4}[args.workload]
    want_cpu = not args.no_cpu_baseline
    wk = make(args.workload, replicas, dev, want_cpu)
    R = wk.replicas
    if args.sequential:
        assert type(wk) is Decode1M and not wk.fp4, "--sequential applies to decode_1m_hierarchical"
        wk.step = wk.step_sequential

    # one eager step per replica (also checks that the library runs)
    for r in range(R):
        wk.step(r)
    torch.cuda.synchronize()

    graphs = None
    if not args.no_graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    wk.step(r)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            wk.step(i % R)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.steps} steps timed: {ms * 1e3:.1f} us per step")

    # the distribution of single steps (an event pair around each replay, a separate pass)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run(i)
        b.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    step_us = {"p10": float(np.percentile(per, 10)), "median": float(np.median(per)),
               "p90": float(np.percentile(per, 90)), "steps": len(per)}

    # a kernel's own time: HIP events around each of its launches (on the stream it is launched on) in
    # eager steps over the same rotated replicas
    def kernel_ms(name, n):
        pairs = []
        for i in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            csa2.csa2_time_next_launch(name, a, b)
            wk.step(i % R)
            if csa2.lib().csa2_timer_pending():  # the step never launched this kernel
                csa2.csa2_time_next_launch(None)
                return None
            pairs.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in pairs]))

    n_eager = min(args.steps, 50)
    kern_ms = kernel_ms(wk.dominant, n_eager)

    alg = wk.algorithmic_bytes()
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded N(0,1), 1% latent channels x20)", "config": wk.config()}
    if isinstance(wk, CedPrefill):
        tf = wk.flops() / (ms * 1e-3) / 1e12
        res.update({"metric": "CED KV projection TFLOP/s (bf16 MFMA, fused FP4 pack) vs MI355X peak",
                    "value": tf, "unit": "TFLOP/s", "dtype": "bf16",
                    "mfma_frac": tf / BF16_PEAK_TFLOPS, "bytes_written_per_step": wk.L * wk.T * (288 + 128)})
        roof = {"bound": "mfma", "achieved": wk.gemm_flops() / (kern_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        qps = wk.queries_per_step / (ms * 1e-3)
        gbps = alg / (ms * 1e-3) / 1e9
        res.update({"value": qps, "unit": "queries/s", "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
                    "algorithmic_bytes_per_step": alg, "queries_per_step": wk.queries_per_step})
        roof = {"bound": "hbm", "achieved": wk.dominant_bytes() / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if getattr(wk, "dominant_flops", lambda: 0)():
        tf = wk.dominant_flops() / (kern_ms * 1e-3) / 1e12
        roof["mfma_tflops"], roof["mfma_frac"] = tf, tf / BF16_PEAK_TFLOPS  # fp16 dense peak = bf16's
    roof["kernel"] = wk.dominant
    roof["kernel_ms"] = kern_ms
    if hasattr(wk, "attn_bytes"):
        # the attention launch of the step: its algorithmic bytes over its own time (latency-bound at batch 1)
        a_ms = kernel_ms("sparse_attn", n_eager)
        c_ms = kernel_ms("attn_combine", n_eager)
        if a_ms:
            ab = wk.attn_bytes()
            res["attn_roofline"] = {"kernel": "sparse_attn", "bound": "hbm", "achieved": ab / (a_ms * 1e-3) / 1e9,
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": ab / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "bytes": ab,
                                    "kernel_ms": a_ms, "combine_ms": c_ms}
    roof["traffic"] = None
    try:  # counter-derived bytes, only while the kernel source is the one they were taken on
        with open(args.traffic_file) as f:
            t = json.load(f).get(f"{args.workload}:{wk.dominant}")
        if t and t.get("source_sha256") == kernel_source_sha(wk.dominant):
            roof["traffic"] = t["bytes_per_launch"]
    except Exception:
        pass
    res["roofline"] = roof
    res["graph"] = graphs is not None
    if args.sequential:
        res["config"]["issue"] = "sequential: one selection and one attention call per layer"
    res["step_us"] = step_us
    # context: what a plain device copy reaches on this GPU (1 GiB read + 1 GiB written)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    res["copy_gbps"] = 5 * 2 * src.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    if want_cpu:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(wk, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
