"""Thin Python binding of libcsa2 (include/csa2.h).

Argument marshalling only: every step of the path runs in the HIP library.
torch supplies device memory and the current stream.  The raw C entry points
are available under their C names on ``lib()``; the helpers below take torch
tensors, allocate outputs with torch and raise ``Csa2Error`` on any status
other than CSA2_OK.  Importing this module never needs a GPU; calling into the
library needs the built libcsa2.so and fails loudly when it is missing.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16, FP4 = 0, 1, 2
FULL, REINDEX = 0, 1
PAGE = 64


class Csa2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)} (status {status})")


class KvLayer(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("rope", ctypes.c_void_p),
        ("idx_keys", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
        ("idx_scales", ctypes.c_void_p),
        ("idx_heads", ctypes.c_int32),
    ]


class Seqs(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class KvFinish(ctypes.Structure):
    """csa2_kv_finish: RMSNorm weights, epsilon, RoPE base and the indexer-key projection."""

    _fields_ = [
        ("gamma", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("w_idx", ctypes.c_void_p),
    ]


class SwaWindow(ctypes.Structure):
    """csa2_swa_window: the FP8 ring of 128 slots per sequence."""

    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("batch", ctypes.c_int32)]


class AppendRowC(ctypes.Structure):
    """csa2_append: one row appended in the scan's launch."""

    _fields_ = [("layer", ctypes.POINTER(KvLayer)), ("latent", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("idx_key", ctypes.c_void_p)]


class ReindexQueryC(ctypes.Structure):
    """csa2_reindex_query: one Reindex layer's query and output."""

    _fields_ = [("q_idx", ctypes.c_void_p), ("w_idx", ctypes.c_void_p), ("indices", ctypes.c_void_p)]


class AttnLayerC(ctypes.Structure):
    """csa2_attn_layer: one layer's attention problem in a multi-layer launch."""

    _fields_ = [("layer", ctypes.POINTER(KvLayer)), ("q", ctypes.c_void_p), ("indices", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("win", ctypes.POINTER(SwaWindow)),
                ("new_latent", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_PKV = ctypes.POINTER(KvLayer)
_PSQ = ctypes.POINTER(Seqs)

# C name -> (restype, argtypes), exactly as declared in include/csa2.h
SIGNATURES = {
    "csa2_abi_version": (ctypes.c_int, []),
    "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa2_time_next_launch": (ctypes.c_int, [ctypes.c_char_p, _P, _P]),
    "csa2_timer_pending": (_I32, []),
    "csa2_debug_checks": (ctypes.c_int, [_I32]),
    "csa2_debug_flags": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
    "csa2_workspace_clear": (ctypes.c_int, [_P, _SZ, _P]),
    "csa2_fp4_pack": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "csa2_fp4_unpack": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P]),
    "csa2_kv_append": (ctypes.c_int, [_PKV, _PSQ, _P, _P, _P, _P]),
    "csa2_ced_kv_project": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "csa2_kv_finish_rows": (ctypes.c_int, [_P, _I64, _I32, _I64, ctypes.POINTER(KvFinish), _P, _P, _P, _P, _P, _P,
                                           _P]),
    "csa2_ced_kv_project_finished": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, ctypes.POINTER(KvFinish), _I64, _P,
                                                    _P, _P, _P, _P, _P]),
    "csa2_kv_append_finished": (ctypes.c_int, [_PKV, _PSQ, _P, ctypes.POINTER(KvFinish), _P]),
    "csa2_swa_append": (ctypes.c_int, [ctypes.POINTER(SwaWindow), _P, _I32, _P, _P]),
    "csa2_swa_attn_merge": (ctypes.c_int, [ctypes.POINTER(SwaWindow), _P, _I32, _P, _I32, _I32, ctypes.c_float, _P,
                                           _P, _P]),
    "csa2_index_scores": (ctypes.c_int, [_PKV, _PSQ, _P, _P, _P, _P]),
    "csa2_topk_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_topk": (ctypes.c_int, [_P, _I64, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "csa2_index_select_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_index_select": (ctypes.c_int, [_PKV, _PSQ, _P, _P, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "csa2_attn_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_sparse_fp4_decode_attn": (ctypes.c_int, [_PKV, _PSQ, _P, _I32, _P, _I32, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "csa2_attn_swa_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_sparse_fp4_decode_attn_swa": (ctypes.c_int, [_PKV, _PSQ, _P, _I32, _P, _I32, ctypes.c_float,
                                                       ctypes.POINTER(SwaWindow), _P, _P, _P, _P, _SZ, _P]),
    "csa2_index_select_append": (ctypes.c_int, [_PKV, _PSQ, ctypes.POINTER(AppendRowC), _I32, _P, _P, _I32, _P, _I32,
                                                _I32, _P, _P, _SZ, _P]),
    "csa2_index_reindex_layers_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_index_reindex_layers": (ctypes.c_int, [_PKV, _PSQ, ctypes.POINTER(ReindexQueryC), _I32, _I32, _P, _I32,
                                                 _I32, _P, _SZ, _P]),
    "csa2_attn_layers_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "csa2_sparse_fp4_decode_attn_layers": (ctypes.c_int, [ctypes.POINTER(AttnLayerC), _I32, _PSQ, _I32, _I32,
                                                          ctypes.c_float, _P, _SZ, _P]),
    "csa2_sparse_fp4_decode_attn_layers_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnLayerC), _I32, _PSQ, _I32,
                                                                  _I32, ctypes.c_float, _P]),
    "csa2_block_pool_create": (_P, [_I32]),
    "csa2_block_alloc": (ctypes.c_int, [_P, _I32, _P]),
    "csa2_block_free": (ctypes.c_int, [_P, _I32, _P]),
    "csa2_block_pool_num_free": (_I32, [_P]),
    "csa2_block_pool_destroy": (None, [_P]),
}

_LIB = None


def lib():
    """The loaded libcsa2 with every declared signature attached."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libcsa2.so is not built ({LIB_PATH}); run `python -m sparse_attention_fp4_kv_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _status_string(s):
    try:
        return lib().csa2_status_string(int(s)).decode()
    except Exception:  # library not loadable: still report the number
        return "status"


def _check(status, where):
    if status != OK:
        raise Csa2Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require(t, dtype, name, device=True):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


# ----------------------------------------------------------------- structures
class PagedLayer:
    """One KV layer's paged pool, allocated with torch on the current device.

    codes [num_blocks*64][256] u8, scales [num_blocks*64][32] u8,
    rope [num_blocks*64][rope_dim] bf16 bits (int16) or None,
    idx_keys [num_blocks*64][64] fp32 / bf16 bits (int16), or for idx_dtype
    "fp4" [num_blocks*64][64] u8 nibbles of 128-dim keys with idx_scales
    [num_blocks*64][8] u8 (scored with idx_heads query heads), or None.
    """

    def __init__(self, num_blocks, rope_dim=0, idx_dtype=None, device="cuda", idx_heads=32):
        rows = num_blocks * PAGE
        self.num_blocks = num_blocks
        self.codes = torch.zeros((rows, 256), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((rows, 32), dtype=torch.uint8, device=device)
        self.rope = torch.zeros((rows, rope_dim), dtype=torch.int16, device=device) if rope_dim else None
        self.rope_dim = rope_dim
        self.idx_dtype = idx_dtype
        if idx_dtype == "f32":
            self.idx_keys = torch.zeros((rows, 64), dtype=torch.float32, device=device)
        elif idx_dtype == "bf16":
            self.idx_keys = torch.zeros((rows, 64), dtype=torch.int16, device=device)
        elif idx_dtype == "fp4":
            self.idx_keys = torch.zeros((rows, 64), dtype=torch.uint8, device=device)
        else:
            self.idx_keys = None
        self.idx_scales = torch.zeros((rows, 8), dtype=torch.uint8, device=device) if idx_dtype == "fp4" else None
        self.idx_heads = idx_heads if idx_dtype == "fp4" else 1

    def struct(self):
        return KvLayer(
            codes=self.codes.data_ptr(), scales=self.scales.data_ptr(),
            rope=self.rope.data_ptr() if self.rope is not None else None,
            idx_keys=self.idx_keys.data_ptr() if self.idx_keys is not None else None,
            num_blocks=self.num_blocks, block_tokens=PAGE, latent_dim=512, rope_dim=self.rope_dim,
            idx_dim=128 if self.idx_dtype == "fp4" else 64,
            idx_dtype={"f32": F32, "fp4": FP4}.get(self.idx_dtype, BF16),
            idx_scales=self.idx_scales.data_ptr() if self.idx_scales is not None else None,
            idx_heads=self.idx_heads)


class Batch:
    """Block tables and lengths of a batch (device int32 tensors)."""

    def __init__(self, block_table, seq_lens, max_seq_len=0):
        _require(block_table, torch.int32, "block_table")
        _require(seq_lens, torch.int32, "seq_lens")
        self.block_table = block_table
        self.seq_lens = seq_lens
        self.max_seq_len = int(max_seq_len)

    @property
    def batch(self):
        return self.block_table.shape[0]

    def struct(self):
        return Seqs(block_table=self.block_table.data_ptr(), max_blocks_per_seq=self.block_table.shape[1],
                    seq_lens=self.seq_lens.data_ptr(), batch=self.block_table.shape[0],
                    max_seq_len=self.max_seq_len)


def workspace(nbytes, device="cuda"):
    """A zeroed workspace of at least nbytes (256-byte aligned by torch's allocator)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- entry points
def csa2_time_next_launch(kernel, start_event=None, stop_event=None):
    """Arm a one-shot HIP-event timing of the next launch of `kernel` (torch.cuda.Event pair)."""
    if kernel is None:
        _check(lib().csa2_time_next_launch(None, None, None), "csa2_time_next_launch")
        return
    for ev in (start_event, stop_event):
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
    _check(lib().csa2_time_next_launch(kernel.encode(), ctypes.c_void_p(start_event.cuda_event),
                                       ctypes.c_void_p(stop_event.cuda_event)), "csa2_time_next_launch")


def csa2_workspace_clear(ws):
    _check(lib().csa2_workspace_clear(_ptr(ws), ws.numel(), _stream()), "csa2_workspace_clear")


def csa2_fp4_pack(x):
    """x: fp32 [rows, C] -> (codes u8 [rows, C/2], scales u8 [rows, C/16])."""
    _require(x, torch.float32, "x")
    rows, C = x.shape
    codes = torch.empty((rows, C // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, C // 16), dtype=torch.uint8, device=x.device)
    _check(lib().csa2_fp4_pack(_ptr(x), rows, C, _ptr(codes), _ptr(scales), _stream()), "csa2_fp4_pack")
    return codes, scales


def csa2_fp4_pack_into(x, codes, scales):
    _require(x, torch.float32, "x")
    rows, C = x.shape
    _check(lib().csa2_fp4_pack(_ptr(x), rows, C, _ptr(codes), _ptr(scales), _stream()), "csa2_fp4_pack")


def csa2_fp4_unpack(codes, scales):
    rows, half = codes.shape
    y = torch.empty((rows, 2 * half), dtype=torch.float32, device=codes.device)
    _check(lib().csa2_fp4_unpack(_ptr(codes), _ptr(scales), rows, 2 * half, _ptr(y), _stream()), "csa2_fp4_unpack")
    return y


def csa2_kv_append(layer, batch, latent, rope=None, idx_key=None):
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_kv_append(ctypes.byref(kv), ctypes.byref(sq), _ptr(latent), _ptr(rope), _ptr(idx_key),
                                _stream()), "csa2_kv_append")


def csa2_ced_kv_project(h, w_kv, w_z=None, c_f32=False):
    """h bf16 bits [T, hidden] (int16); w_kv [L, 512, hidden]; w_z [L, 64, hidden] or None."""
    T, hidden = h.shape
    L = w_kv.shape[0]
    dev = h.device
    codes = torch.empty((L, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((L, T, 32), dtype=torch.uint8, device=dev)
    z = torch.empty((L, T, 64), dtype=torch.int16, device=dev) if w_z is not None else None
    c = torch.empty((L, T, 512), dtype=torch.float32, device=dev) if c_f32 else None
    _check(lib().csa2_ced_kv_project(_ptr(h), T, hidden, L, _ptr(w_kv), _ptr(w_z), _ptr(codes), _ptr(scales), _ptr(z),
                                     _ptr(c), _stream()), "csa2_ced_kv_project")
    return codes, scales, z, c


def _finish(gamma, eps, theta, w_idx):
    _require(gamma, torch.float32, "gamma")
    return KvFinish(gamma=gamma.data_ptr(), eps=eps, rope_theta=theta,
                    w_idx=w_idx.data_ptr() if w_idx is not None else None)


def csa2_kv_finish_rows(c, gamma, eps, theta, w_idx=None, pos0=0, debug=False):
    """c fp32 [L, T, 512] raw latents; gamma fp32 [L, 512]; w_idx bf16 bits [L, 128, 512] (int16) or None.

    Returns (codes [L,T,256], scales [L,T,32], idx_codes [L,T,64] | None, idx_scales [L,T,8] | None,
    x_f32 [L,T,512] | None, k_f32 [L,T,128] | None); the fp32 copies only with debug."""
    _require(c, torch.float32, "c")
    L, T, _ = c.shape
    dev = c.device
    codes = torch.empty((L, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((L, T, 32), dtype=torch.uint8, device=dev)
    kc = torch.empty((L, T, 64), dtype=torch.uint8, device=dev) if w_idx is not None else None
    ks = torch.empty((L, T, 8), dtype=torch.uint8, device=dev) if w_idx is not None else None
    x = torch.empty((L, T, 512), dtype=torch.float32, device=dev) if debug else None
    k = torch.empty((L, T, 128), dtype=torch.float32, device=dev) if debug and w_idx is not None else None
    fin = _finish(gamma, eps, theta, w_idx)
    _check(lib().csa2_kv_finish_rows(_ptr(c), T, L, pos0, ctypes.byref(fin), _ptr(codes), _ptr(scales), _ptr(kc),
                                     _ptr(ks), _ptr(x), _ptr(k), _stream()), "csa2_kv_finish_rows")
    return codes, scales, kc, ks, x, k


def csa2_ced_kv_project_finished(h, w_kv, gamma, eps, theta, w_idx=None, pos0=0):
    """CED projection followed by the finish; returns (codes, scales, idx_codes | None, idx_scales | None, c_f32)."""
    T, hidden = h.shape
    L = w_kv.shape[0]
    dev = h.device
    c = torch.empty((L, T, 512), dtype=torch.float32, device=dev)
    codes = torch.empty((L, T, 256), dtype=torch.uint8, device=dev)
    scales = torch.empty((L, T, 32), dtype=torch.uint8, device=dev)
    kc = torch.empty((L, T, 64), dtype=torch.uint8, device=dev) if w_idx is not None else None
    ks = torch.empty((L, T, 8), dtype=torch.uint8, device=dev) if w_idx is not None else None
    fin = _finish(gamma, eps, theta, w_idx)
    _check(lib().csa2_ced_kv_project_finished(_ptr(h), T, hidden, L, _ptr(w_kv), ctypes.byref(fin), pos0, _ptr(c),
                                              _ptr(codes), _ptr(scales), _ptr(kc), _ptr(ks), _stream()),
           "csa2_ced_kv_project_finished")
    return codes, scales, kc, ks, c


def csa2_kv_append_finished(layer, batch, latent, gamma, eps, theta, w_idx=None):
    """Raw latent fp32 [B, 512] finished into the slot of position seq_lens[b]; gamma [512], w_idx [128, 512]."""
    kv, sq = layer.struct(), batch.struct()
    fin = _finish(gamma, eps, theta, w_idx)
    _check(lib().csa2_kv_append_finished(ctypes.byref(kv), ctypes.byref(sq), _ptr(latent), ctypes.byref(fin),
                                         _stream()), "csa2_kv_append_finished")


class SwaRing:
    """Sliding-window ring of one layer: codes [batch][128][512] u8 (E4M3FN), scales [batch][128] fp32."""

    def __init__(self, batch, device="cuda"):
        self.codes = torch.zeros((batch, 128, 512), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((batch, 128), dtype=torch.float32, device=device)
        self.batch = batch

    def struct(self):
        return SwaWindow(codes=self.codes.data_ptr(), scales=self.scales.data_ptr(), batch=self.batch)


def csa2_swa_append(ring, positions, latent):
    """positions int32 [B] (device), latent fp32 [B, 512]."""
    w = ring.struct()
    _check(lib().csa2_swa_append(ctypes.byref(w), _ptr(positions), latent.shape[0], _ptr(latent), _stream()),
           "csa2_swa_append")


def csa2_swa_attn_merge(ring, seq_lens, q, softmax_scale, out, lse):
    """Merges the window attention into (out [B, H, 512], lse [B, H]) in place; q bf16 bits [B, H, 512 (+64)]."""
    B, H, D = q.shape
    w = ring.struct()
    _check(lib().csa2_swa_attn_merge(ctypes.byref(w), _ptr(seq_lens), B, _ptr(q), H, D, softmax_scale, _ptr(out),
                                     _ptr(lse), _stream()), "csa2_swa_attn_merge")


def csa2_index_scores(layer, batch, q_idx, max_len, w_idx=None):
    """q_idx fp32 [B, 64] (fp32 / bf16 keys) or fp16 [B, heads, 128] with w_idx fp32 [B, heads] (FP4 keys)."""
    scores = torch.empty((batch.batch, max_len), dtype=torch.float32, device=q_idx.device)
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_index_scores(ctypes.byref(kv), ctypes.byref(sq), _ptr(q_idx), _ptr(w_idx), _ptr(scores),
                                   _stream()), "csa2_index_scores")
    return scores


def topk_workspace_bytes(batch, max_len, top_k):
    n = ctypes.c_size_t()
    _check(lib().csa2_topk_workspace_size(batch, max_len, top_k, ctypes.byref(n)), "csa2_topk_workspace_size")
    return n.value


def csa2_topk(scores, lens, top_k, ws=None):
    _require(scores, torch.float32, "scores")
    B, M = scores.shape
    if ws is None:
        ws = workspace(topk_workspace_bytes(B, M, top_k), scores.device)
    idx = torch.empty((B, top_k), dtype=torch.int32, device=scores.device)
    _check(lib().csa2_topk(_ptr(scores), M, _ptr(lens), B, M, top_k, _ptr(idx), _ptr(ws), ws.numel(), _stream()),
           "csa2_topk")
    return idx


def index_select_workspace_bytes(batch, max_len, top_k, pool_blocks=0):
    n = ctypes.c_size_t()
    _check(lib().csa2_index_select_workspace_size(batch, max_len, top_k, pool_blocks, 8 if pool_blocks else 0,
                                                  ctypes.byref(n)), "csa2_index_select_workspace_size")
    return n.value


def csa2_index_select(layer, batch, q_idx, top_k, mode=FULL, pool_in=None, pool_blocks=0, want_pool=False,
                      ws=None, indices=None, pool_out=None, w_idx=None):
    """Full (optionally hierarchical: want_pool) or Reindex selection -> (indices, pool_out or None)."""
    B = batch.batch
    dev = q_idx.device
    max_len = batch.max_seq_len or batch.block_table.shape[1] * PAGE
    pooled = mode == REINDEX or want_pool
    if ws is None:
        ws = workspace(index_select_workspace_bytes(B, max_len, top_k, pool_blocks if pooled else 0), dev)
    if indices is None:
        indices = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    if want_pool and pool_out is None:
        pool_out = torch.empty((B, pool_blocks), dtype=torch.int32, device=dev)
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_index_select(ctypes.byref(kv), ctypes.byref(sq), _ptr(q_idx), _ptr(w_idx), top_k, mode,
                                   _ptr(pool_in),
                                   _ptr(pool_out) if want_pool else None, pool_blocks, 8 if pooled else 0,
                                   _ptr(indices), _ptr(ws), ws.numel(), _stream()), "csa2_index_select")
    return indices, (pool_out if want_pool else None)


def attn_workspace_bytes(batch, heads, top_k):
    n = ctypes.c_size_t()
    _check(lib().csa2_attn_workspace_size(batch, heads, top_k, 512, ctypes.byref(n)), "csa2_attn_workspace_size")
    return n.value


def csa2_sparse_fp4_decode_attn(layer, batch, q, indices, softmax_scale, ws=None, out=None, lse=None):
    """q bf16 bits [B, H, 512+rope] (int16); indices int32 [B, K] -> (out fp32 [B, H, 512], lse fp32 [B, H])."""
    B, H, _ = q.shape
    K = indices.shape[1]
    dev = q.device
    if ws is None:
        ws = workspace(attn_workspace_bytes(B, H, K), dev)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_sparse_fp4_decode_attn(ctypes.byref(kv), ctypes.byref(sq), _ptr(q), H, _ptr(indices), K,
                                             float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                             _stream()), "csa2_sparse_fp4_decode_attn")
    return out, lse


def attn_swa_workspace_bytes(batch, heads, top_k):
    n = ctypes.c_size_t()
    _check(lib().csa2_attn_swa_workspace_size(batch, heads, top_k, 512, ctypes.byref(n)),
           "csa2_attn_swa_workspace_size")
    return n.value


def csa2_sparse_fp4_decode_attn_swa(layer, batch, q, indices, softmax_scale, ring, new_latent=None, ws=None, out=None,
                                    lse=None):
    """csa2_sparse_fp4_decode_attn with the sliding-window ring in the same softmax -> (out, lse).

    new_latent: fp32 [B, 512] (device), the current token's window entry appended in the same call, or None."""
    B, H, _ = q.shape
    K = indices.shape[1]
    dev = q.device
    if ws is None:
        ws = workspace(attn_swa_workspace_bytes(B, H, K), dev)
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    kv, sq, w = layer.struct(), batch.struct(), ring.struct()
    _check(lib().csa2_sparse_fp4_decode_attn_swa(ctypes.byref(kv), ctypes.byref(sq), _ptr(q), H, _ptr(indices), K,
                                                 float(softmax_scale), ctypes.byref(w), _ptr(new_latent), _ptr(out),
                                                 _ptr(lse),
                                                 _ptr(ws), ws.numel(), _stream()), "csa2_sparse_fp4_decode_attn_swa")
    return out, lse


def csa2_index_select_append(layer, batch, q_idx, top_k, appends, pool_blocks=0, want_pool=False, ws=None,
                             indices=None, pool_out=None, w_idx=None):
    """Full selection (optionally with the pool) over seq_lens positions, with this step's rows appended at
    position seq_lens[b] - 1 in the same launch.  appends: list of (layer, latent | None, rope | None,
    idx_key | None) -> (indices, pool_out or None)."""
    B = batch.batch
    dev = q_idx.device
    max_len = batch.max_seq_len or batch.block_table.shape[1] * PAGE
    if ws is None:
        ws = workspace(index_select_workspace_bytes(B, max_len, top_k, pool_blocks if want_pool else 0), dev)
    if indices is None:
        indices = torch.empty((B, top_k), dtype=torch.int32, device=dev)
    if want_pool and pool_out is None:
        pool_out = torch.empty((B, pool_blocks), dtype=torch.int32, device=dev)
    kvs = [a[0].struct() for a in appends]  # kept alive for the call
    rows = (AppendRowC * max(len(appends), 1))(
        *[AppendRowC(ctypes.pointer(kv), _ptr(a[1]), _ptr(a[2]), _ptr(a[3])) for kv, a in zip(kvs, appends)])
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_index_select_append(ctypes.byref(kv), ctypes.byref(sq), rows, len(appends), _ptr(q_idx),
                                          _ptr(w_idx), top_k, _ptr(pool_out) if want_pool else None, pool_blocks,
                                          8 if want_pool else 0, _ptr(indices), _ptr(ws), ws.numel(), _stream()),
           "csa2_index_select_append")
    return indices, (pool_out if want_pool else None)


def reindex_layers_workspace_bytes(n_layers, batch, top_k, pool_blocks):
    n = ctypes.c_size_t()
    _check(lib().csa2_index_reindex_layers_workspace_size(n_layers, batch, top_k, pool_blocks, 8, ctypes.byref(n)),
           "csa2_index_reindex_layers_workspace_size")
    return n.value


def csa2_index_reindex_layers(layer, batch, queries, top_k, pool_in, pool_blocks, ws=None, indices=None):
    """Reindex of several layers over one pool.  queries: list of (q_idx, w_idx | None); indices: list of
    int32 [B, K] outputs or None -> list of indices."""
    B = batch.batch
    dev = pool_in.device
    L = len(queries)
    if ws is None:
        ws = workspace(reindex_layers_workspace_bytes(L, B, top_k, pool_blocks), dev)
    if indices is None:
        indices = [torch.empty((B, top_k), dtype=torch.int32, device=dev) for _ in range(L)]
    qs = (ReindexQueryC * L)(*[ReindexQueryC(_ptr(q), _ptr(w), _ptr(o)) for (q, w), o in zip(queries, indices)])
    kv, sq = layer.struct(), batch.struct()
    _check(lib().csa2_index_reindex_layers(ctypes.byref(kv), ctypes.byref(sq), qs, L, top_k, _ptr(pool_in),
                                           pool_blocks, 8, _ptr(ws), ws.numel(), _stream()),
           "csa2_index_reindex_layers")
    return indices


def attn_layers_workspace_bytes(n_layers, batch, heads, top_k, window=False):
    n = ctypes.c_size_t()
    _check(lib().csa2_attn_layers_workspace_size(n_layers, batch, heads, top_k, 512, 1 if window else 0,
                                                 ctypes.byref(n)), "csa2_attn_layers_workspace_size")
    return n.value


def csa2_sparse_fp4_decode_attn_layers(jobs, batch, softmax_scale, ws=None, outs=None, lses=None):
    """Several layers' attention in one launch.  jobs: list of (layer, q bf16 bits [B, H, 512+rope], indices
    int32 [B, K]) or (layer, q, indices, ring, new_latent | None) with a sliding window -> (outs, lses)."""
    B, H, _ = jobs[0][1].shape
    K = jobs[0][2].shape[1]
    dev = jobs[0][1].device
    L = len(jobs)
    window = len(jobs[0]) > 3
    if ws is None:
        ws = workspace(attn_layers_workspace_bytes(L, B, H, K, window), dev)
    if outs is None:
        outs = [torch.empty((B, H, 512), dtype=torch.float32, device=dev) for _ in range(L)]
    if lses is None:
        lses = [torch.empty((B, H), dtype=torch.float32, device=dev) for _ in range(L)]
    kvs = [j[0].struct() for j in jobs]  # kept alive for the call
    wins = [j[3].struct() if window else None for j in jobs]
    arr = (AttnLayerC * L)(*[
        AttnLayerC(ctypes.pointer(kv), _ptr(j[1]), _ptr(j[2]), _ptr(o), _ptr(ls),
                   ctypes.pointer(w) if w is not None else None, _ptr(j[4]) if window else None)
        for kv, w, j, o, ls in zip(kvs, wins, jobs, outs, lses)])
    sq = batch.struct()
    _check(lib().csa2_sparse_fp4_decode_attn_layers(arr, L, ctypes.byref(sq), H, K, float(softmax_scale), _ptr(ws),
                                                    ws.numel(), _stream()), "csa2_sparse_fp4_decode_attn_layers")
    return outs, lses


DBG_Q_RANGE, DBG_INDEX, DBG_PAGE, DBG_NONFINITE, DBG_SCORE, DBG_SEQ_LEN = 1, 2, 4, 8, 16, 32


def csa2_debug_checks(enable):
    _check(lib().csa2_debug_checks(1 if enable else 0), "csa2_debug_checks")


def csa2_debug_flags():
    """Waits for the device; returns and clears the debug bits raised since the last call."""
    v = ctypes.c_uint32()
    _check(lib().csa2_debug_flags(ctypes.byref(v)), "csa2_debug_flags")
    return v.value


class BlockPool:
    """Host-side page allocator (csa2_block_pool_*)."""

    def __init__(self, num_blocks):
        self._h = lib().csa2_block_pool_create(num_blocks)
        if not self._h:
            raise Csa2Error(ERR_INVALID_ARG, "csa2_block_pool_create")

    def alloc(self, n):
        arr = (ctypes.c_int32 * max(n, 1))()
        _check(lib().csa2_block_alloc(self._h, n, arr), "csa2_block_alloc")
        return [arr[i] for i in range(n)]

    def free(self, ids):
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        _check(lib().csa2_block_free(self._h, len(ids), arr), "csa2_block_free")

    @property
    def num_free(self):
        return lib().csa2_block_pool_num_free(self._h)

    def close(self):
        if self._h:
            lib().csa2_block_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
