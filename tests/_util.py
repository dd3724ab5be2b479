"""Helpers shared by the GPU parity tests: cache construction from the seeded
inputs and the comparison rules.

Comparison rules (fixed before any kernel was written):
  * packing, pools of equal scores, integer work: bit-exact;
  * top-K sets: equal, except positions whose oracle score lies within
    1e-5 * max(|S_K|, rms(scores)) of the K-th oracle score S_K;
  * attention: max |out - oracle| <= 2e-3 (fp32 accumulation), lse <= 1e-3.
"""

import numpy as np
import torch

import oracle
from sparse_attention_fp4_kv_amd import csa2, workloads as wl

ATTN_TOL = 2e-3
LSE_TOL = 1e-3
TOPK_REL = 1e-5


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a).to(dev())
    return t if dtype is None else t.to(dtype)


def build_tables(st, seq_lens, permuted, extra_blocks=0):
    tables, nb = wl.block_tables(st, seq_lens, permuted, extra_blocks)
    return tables, nb


def fill_layer(layer, tables, seq_lens, latents=None, keys=None, ropes=None):
    """Write per-sequence arrays into the paged pool at the table's physical rows.

    latents[b]: fp32 [n_b][512] (packed on the GPU); keys[b]: fp32 or bf16 bits
    [n_b][64], or for an FP4 layer fp32 [n_b][128] (packed on the GPU);
    ropes[b]: bf16 bits [n_b][64].
    """
    for b, n in enumerate(seq_lens):
        if n == 0:
            continue
        rows = oracle.paged.physical_rows(tables[b], np.arange(n))
        rows_t = torch.from_numpy(rows).to(dev())
        if latents is not None:
            codes, scales = csa2.csa2_fp4_pack(to_dev(latents[b]))
            layer.codes[rows_t] = codes
            layer.scales[rows_t] = scales
        if keys is not None and layer.idx_dtype == "fp4":
            codes, scales = csa2.csa2_fp4_pack(to_dev(keys[b]))
            layer.idx_keys[rows_t] = codes
            layer.idx_scales[rows_t] = scales
        elif keys is not None:
            layer.idx_keys[rows_t] = to_dev(keys[b])
        if ropes is not None:
            layer.rope[rows_t] = to_dev(ropes[b])
    torch.cuda.synchronize()


def make_batch(tables, seq_lens, max_len=0):
    return csa2.Batch(to_dev(tables.astype(np.int32)), to_dev(np.asarray(seq_lens, dtype=np.int32)), max_len)


def topk_tolerance(scores):
    scores = np.asarray(scores, dtype=np.float64)
    return lambda sk: TOPK_REL * max(abs(sk), float(np.sqrt(np.mean(scores ** 2))) if scores.size else 0.0)


def check_topk(gpu_row, score_of, k, where=""):
    """gpu_row: int array [k] (-1 padded); score_of: dict position -> oracle score (all candidates)."""
    gpu = [int(i) for i in gpu_row if i >= 0]
    assert len(gpu) == len(set(gpu)), f"{where}: duplicate indices"
    assert all(i in score_of for i in gpu), f"{where}: index outside the candidates"
    pos = np.array(list(score_of.keys()), dtype=np.int64)
    sc = np.array([score_of[p] for p in pos], dtype=np.float64)
    ref = oracle.indexer.topk(sc, k, positions=pos)
    ref_set = set(int(i) for i in ref if i >= 0)
    assert len(gpu) == len(ref_set), f"{where}: {len(gpu)} selected, oracle {len(ref_set)}"
    assert int(np.sum(np.asarray(gpu_row) < 0)) == k - len(ref_set), f"{where}: wrong -1 padding"
    diff = ref_set.symmetric_difference(gpu)
    if diff:
        sk = min(score_of[i] for i in ref_set)
        tol = topk_tolerance(sc)(sk)
        bad = [i for i in diff if abs(score_of[i] - sk) > tol]
        assert not bad, f"{where}: {len(diff)} differing indices, {len(bad)} beyond tolerance (S_K={sk})"
    return len(diff)


def oracle_attention_rows(latent, ropes, q_bits, sel, n, sigma):
    """Oracle attention of one sequence: latent fp32 [n][512], sel positions, rope bits or None."""
    valid = oracle.attention.valid_slots(sel, n)
    codes, scales = oracle.fp4.fp4_pack(latent[valid]) if len(valid) else (np.zeros((0, 256), np.uint8),
                                                                          np.zeros((0, 32), np.uint8))
    c = oracle.fp4.fp4_unpack(codes, scales)
    rope = oracle.ced.bf16_bits_to_f64(ropes[valid]) if ropes is not None else None
    return oracle.attention.sparse_attention(q_bits, c, sigma, rope_sel=rope)


def pack_close(codes_g, scales_g, x_ref, rel=1e-5, abs_=1e-6, tol=None):
    """FP4 bytes from the GPU (codes [n][C/2], scales [n][C/16]) against the oracle's pack of x_ref
    (float64 [n][C], computed by the oracle in exact arithmetic): a group may differ only where x_ref
    sits within its tolerance of a decision point (the scale's rounding boundary or an element
    threshold), or a differing sign belongs to a value within its tolerance of zero.  The tolerance of
    element i is rel * |x_i| + abs_, plus tol[i] when an array tol (same shape as x_ref, absolute) is
    given.  Returns the number of differing groups."""
    fp4 = oracle.fp4
    x = np.asarray(x_ref, dtype=np.float64)
    n, C = x.shape
    t_all = rel * np.abs(x) + abs_
    if tol is not None:
        t_all = t_all + np.broadcast_to(np.asarray(tol, dtype=np.float64), x.shape)
    oc, os_ = fp4.fp4_pack(x.astype(np.float32))
    codes_g, scales_g = np.asarray(codes_g), np.asarray(scales_g)

    def nibbles(c):
        return np.stack([c & 0xF, c >> 4], axis=-1).reshape(n, C).astype(np.int64)

    ng, no = nibbles(codes_g), nibbles(oc)
    gd = (scales_g != os_) | np.any((ng != no).reshape(n, C // 16, 16), axis=-1)
    for r, g in zip(*np.nonzero(gd)):
        xs = x[r, 16 * g:16 * g + 16]
        ts = t_all[r, 16 * g:16 * g + 16]
        sg = int(scales_g[r, g])
        if sg != int(os_[r, g]):
            # any code between the scales of the smallest and largest amax the tolerance allows
            a_lo = float(np.max(np.maximum(np.abs(xs) - ts, 0.0)))
            a_hi = float(np.max(np.abs(xs) + ts))
            lo_c = int(fp4.e4m3_encode(np.float64(a_lo / 6)))
            hi_c = int(fp4.e4m3_encode(np.float64(a_hi / 6)))
            assert lo_c <= sg <= hi_c, f"row {r} group {g}: scale {sg:#x}, oracle {int(os_[r, g]):#x}, amax in [{a_lo}, {a_hi}]"
        s = float(fp4.e4m3_decode(np.uint8(sg)))
        for i in np.nonzero(ng[r, 16 * g:16 * g + 16] != (no[r, 16 * g:16 * g + 16] if sg == int(os_[r, g]) else -1))[0]:
            v, t = xs[i], ts[i]
            got = int(ng[r, 16 * g + i])
            if s == 0:
                assert got == 0, f"row {r} group {g}: nibble {got:#x} under a zero scale"
                continue
            lo = int(fp4.e2m1_quantize_magnitude(max(abs(v) - t, 0.0), s))
            hi = int(fp4.e2m1_quantize_magnitude(abs(v) + t, s))
            assert lo <= (got & 7) <= hi, f"row {r} group {g} elem {i}: nibble {got:#x}, value {v}, scale {s}"
            assert (got >> 3) == int(np.signbit(v)) or abs(v) <= t, f"row {r} group {g} elem {i}: sign"
    return int(np.sum(gd))
