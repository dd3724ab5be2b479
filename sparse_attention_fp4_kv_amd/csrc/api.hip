// C ABI of libcsa2: argument validation, launch dispatch, workspace sizing
// and the host-side page allocator.  Every public entry point validates its
// arguments before launching anything and never lets a C++ exception out.
#include "../../include/csa2.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "kernels.h"

using namespace csa2;

namespace {
// roctx ranges around every call that launches work, named after the call,
// for profilers (rocprofv3 --marker-trace); on when the environment variable
// CSA2_ROCTX is set to a nonzero value, read once.
bool roctx_on() {
  static const bool on = [] {
    const char *e = std::getenv("CSA2_ROCTX");
    return e != nullptr && std::atoi(e) != 0;
  }();
  return on;
}
struct TraceRange {
  bool on;
  explicit TraceRange(const char *name) : on(roctx_on()) {
    if (on) roctxRangePushA(name);
  }
  ~TraceRange() {
    if (on) roctxRangePop();
  }
  TraceRange(const TraceRange &) = delete;
  TraceRange &operator=(const TraceRange &) = delete;
};
}  // namespace
#define CSA2_TRACE TraceRange trace_range_(__func__)

// The debug flag word of every device (word 0 is used; the rest pads it to
// its own cache line).
static __device__ __align__(256) uint32_t dbg_word[64];

namespace {
std::atomic<int> g_debug{-1};  // -1: the environment has not been read yet
std::mutex g_dbg_mu;
void *g_dbg_addr[kMaxDevices] = {};

bool debug_on() {
  int v = g_debug.load();
  if (v < 0) {
    const char *e = std::getenv("CSA2_DEBUG_CHECKS");
    int want = (e != nullptr && std::atoi(e) != 0) ? 1 : 0;
    g_debug.compare_exchange_strong(v, want);
    v = g_debug.load();
  }
  return v > 0;
}

// The flag word's address on the current device (resolved once per device).
void *dbg_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (g_dbg_addr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_word)) != hipSuccess) return nullptr;
    g_dbg_addr[dev] = p;
  }
  return g_dbg_addr[dev];
}
}  // namespace

namespace csa2 {
uint32_t *debug_flags() { return debug_on() ? static_cast<uint32_t *>(dbg_address()) : nullptr; }
}  // namespace csa2

namespace {

constexpr int kMaxTopK = 4096;
constexpr int kMaxPoolBlocks = 2048;  // pool positions must fit one 16,384-candidate select
constexpr int64_t kMaxSelectLen = 4096LL * 2048;  // 8M positions per row
// Sequences per call, and (layer, sequence) problems per layered attention
// launch: each spans one grid dimension, which also keeps the host's int
// products of these counts with heads and splits in range.
constexpr int32_t kMaxBatch = 65535;

hipStream_t as_stream(csa2_stream s) { return reinterpret_cast<hipStream_t>(s); }

csa2_status from_hip(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Indexer keys of a layer: 64-dim fp32 / bf16 with one query head, or 128-dim
// FP4 (nibbles + E4M3 scales) with 1 .. 32 query heads.
bool keys_ok(const csa2_kv_layer *l) {
  if (l->idx_keys == nullptr || !aligned(l->idx_keys, 16)) return false;
  if (l->idx_dtype == CSA2_F32 || l->idx_dtype == CSA2_BF16) return l->idx_dim == 64 && l->idx_heads == 1;
  if (l->idx_dtype != CSA2_FP4) return false;
  return l->idx_dim == 128 && l->idx_heads >= 1 && l->idx_heads <= 32 && l->idx_scales != nullptr &&
         aligned(l->idx_scales, 8);
}

// Checks a layer and produces its device view.  need_kv: codes/scales are read;
// need_keys: idx_keys are read.
csa2_status check_layer(const csa2_kv_layer *l, bool need_kv, bool need_keys, KvLayerDev *out) {
  if (l == nullptr) return CSA2_ERR_INVALID_ARG;
  if (l->block_tokens != 64 || l->latent_dim != 512 || l->num_blocks < 0) return CSA2_ERR_INVALID_ARG;
  if (l->num_blocks > (1 << 25)) return CSA2_ERR_INVALID_ARG;  // rows are addressed with 32-bit indices
  if (l->rope_dim != 0 && l->rope_dim != 64) return CSA2_ERR_INVALID_ARG;
  if (need_kv) {
    if (l->codes == nullptr || l->scales == nullptr) return CSA2_ERR_INVALID_ARG;
    if (!aligned(l->codes, 16) || !aligned(l->scales, 16)) return CSA2_ERR_INVALID_ARG;
    if (l->rope_dim != 0 && (l->rope == nullptr || !aligned(l->rope, 16))) return CSA2_ERR_INVALID_ARG;
  }
  if (need_keys && !keys_ok(l)) return CSA2_ERR_INVALID_ARG;
  out->codes = l->codes;
  out->scales = l->scales;
  out->rope = l->rope_dim ? l->rope : nullptr;
  out->idx_keys = l->idx_keys;
  out->idx_scales = l->idx_dtype == CSA2_FP4 ? l->idx_scales : nullptr;
  out->num_blocks = l->num_blocks;
  out->rope_dim = l->rope_dim;
  out->idx_f32 = l->idx_dtype == CSA2_F32 ? 1 : 0;
  out->idx_fp4 = l->idx_dtype == CSA2_FP4 ? 1 : 0;
  out->idx_heads = l->idx_dtype == CSA2_FP4 ? l->idx_heads : 1;
  return CSA2_OK;
}

// The query of an indexer call matches the keys' kind: fp32 [B][64] and no
// weights for fp32 / bf16 keys, fp16 heads and fp32 weights for FP4 keys.
bool query_ok(const csa2_kv_layer *l, const void *q_idx, const float *w_idx) {
  if (q_idx == nullptr) return false;
  if (l->idx_dtype == CSA2_FP4) return w_idx != nullptr && aligned(q_idx, 16) && aligned(w_idx, 4);
  return w_idx == nullptr && aligned(q_idx, 4);
}

csa2_status check_seqs(const csa2_seqs *s, SeqsDev *out) {
  if (s == nullptr || s->batch < 0 || s->batch > kMaxBatch || s->max_blocks_per_seq < 0 || s->max_seq_len < 0)
    return CSA2_ERR_INVALID_ARG;
  if (s->batch > 0 && (s->block_table == nullptr || s->seq_lens == nullptr)) return CSA2_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)s->max_blocks_per_seq * 64;
  const int64_t ml = s->max_seq_len ? s->max_seq_len : cap;
  if (ml > cap || ml > kMaxSelectLen) return CSA2_ERR_INVALID_ARG;
  out->block_table = s->block_table;
  out->seq_lens = s->seq_lens;
  out->max_blocks = s->max_blocks_per_seq;
  out->batch = s->batch;
  out->max_len = (int)ml;
  return CSA2_OK;
}

// One-shot launch timer armed by csa2_time_next_launch.
struct ArmedTimer {
  int id = -1;
  hipEvent_t start = nullptr, stop = nullptr;
  bool started = false;
};
ArmedTimer g_timer;

const char *const kKernelNames[kKernCount] = {"index_scan",  "pool_score",   "topk_given", "topk_compact",
                                              "sparse_attn", "attn_combine", "ced_project", "fp4_pack",
                                              "kv_append",   "index_scores", "kv_finish",    "swa_attn"};

}  // namespace

namespace csa2 {
void timer_before(KernelId id, hipStream_t st) {
  if (g_timer.id != (int)id || g_timer.started) return;
  if (hipEventRecord(g_timer.start, st) == hipSuccess) g_timer.started = true;
}
void timer_after(KernelId id, hipStream_t st) {
  if (g_timer.id != (int)id || !g_timer.started) return;
  (void)hipEventRecord(g_timer.stop, st);
  g_timer = ArmedTimer();
}
}  // namespace csa2

struct csa2_block_pool {
  std::vector<int32_t> free_ids;   // stack of free ids
  std::vector<uint8_t> is_free;    // per id
};

extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char *csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

csa2_status csa2_time_next_launch(const char *kernel, void *start_event, void *stop_event) {
  if (kernel == nullptr) {
    g_timer = ArmedTimer();
    return CSA2_OK;
  }
  if (start_event == nullptr || stop_event == nullptr) return CSA2_ERR_INVALID_ARG;
  for (int i = 0; i < kKernCount; ++i) {
    if (std::strcmp(kernel, kKernelNames[i]) == 0) {
      g_timer.id = i;
      g_timer.start = static_cast<hipEvent_t>(start_event);
      g_timer.stop = static_cast<hipEvent_t>(stop_event);
      g_timer.started = false;
      return CSA2_OK;
    }
  }
  return CSA2_ERR_INVALID_ARG;
}

int32_t csa2_timer_pending(void) { return g_timer.id >= 0 ? 1 : 0; }

csa2_status csa2_debug_checks(int32_t enable) {
  g_debug.store(enable != 0 ? 1 : 0);
  if (enable != 0 && dbg_address() == nullptr) return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_debug_flags(uint32_t *flags) {
  if (flags == nullptr) return CSA2_ERR_INVALID_ARG;
  *flags = 0;
  void *p = dbg_address();
  if (p == nullptr) return CSA2_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return CSA2_ERR_HIP;
  const uint32_t zero = 0;
  if (hipMemcpy(flags, p, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return CSA2_ERR_HIP;
  if (hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_workspace_clear(void *ws, size_t bytes, csa2_stream stream) {
  CSA2_TRACE;
  if (bytes == 0) return CSA2_OK;
  if (ws == nullptr || !aligned(ws, 4) || bytes % 4 != 0) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_fill_zero(ws, bytes, as_stream(stream)));
}

csa2_status csa2_fp4_pack(const float *x, int64_t rows, int32_t channels, uint8_t *codes, uint8_t *scales,
                          csa2_stream stream) {
  CSA2_TRACE;
  if (rows < 0 || channels <= 0 || channels % 16 != 0) return CSA2_ERR_INVALID_ARG;
  if (rows == 0) return CSA2_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_fp4_pack(x, rows, channels, codes, scales, as_stream(stream)));
}

csa2_status csa2_fp4_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t channels, float *y,
                            csa2_stream stream) {
  CSA2_TRACE;
  if (rows < 0 || channels <= 0 || channels % 16 != 0) return CSA2_ERR_INVALID_ARG;
  if (rows == 0) return CSA2_OK;
  if (y == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(codes, 8)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_fp4_unpack(codes, scales, rows, channels, y, as_stream(stream)));
}

csa2_status csa2_kv_append(const csa2_kv_layer *layer, const csa2_seqs *seqs, const float *latent,
                           const uint16_t *rope, const void *idx_key, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(layer, latent != nullptr, false, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (S.batch == 0) return CSA2_OK;
  if (latent == nullptr && rope == nullptr && idx_key == nullptr) return CSA2_ERR_INVALID_ARG;
  if (rope != nullptr && (L.rope_dim == 0 || layer->rope == nullptr)) return CSA2_ERR_INVALID_ARG;
  if (latent != nullptr && L.rope_dim != 0 && rope == nullptr) return CSA2_ERR_INVALID_ARG;
  if (idx_key != nullptr && !keys_ok(layer)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_kv_append(L, S, latent, rope, idx_key, as_stream(stream)));
}

namespace {
csa2_status check_finish(const csa2_kv_finish *fin, csa2::KvFinish *out) {
  if (fin == nullptr || fin->gamma == nullptr || !aligned(fin->gamma, 16)) return CSA2_ERR_INVALID_ARG;
  if (!(fin->eps > 0.0f) || !(fin->eps < 3.0e38f)) return CSA2_ERR_INVALID_ARG;
  if (!(fin->rope_theta >= 0.0f) || !(fin->rope_theta < 3.0e38f)) return CSA2_ERR_INVALID_ARG;
  if (fin->w_idx != nullptr && !aligned(fin->w_idx, 16)) return CSA2_ERR_INVALID_ARG;
  *out = csa2::KvFinish{fin->gamma, fin->eps, fin->rope_theta, fin->w_idx};
  return CSA2_OK;
}

csa2_status check_finish_rows(int64_t tokens, int32_t n_layers, int64_t pos0, const csa2_kv_finish *fin,
                              uint8_t *codes, uint8_t *scales, uint8_t *idx_codes, uint8_t *idx_scales,
                              const float *x_f32, const float *k_f32, csa2::KvFinish *f) {
  if (tokens < 0 || n_layers < 0 || n_layers > 4096 || pos0 < 0) return CSA2_ERR_INVALID_ARG;
  if (pos0 + tokens > ((int64_t)1 << 24)) return CSA2_ERR_INVALID_ARG;
  csa2_status st = check_finish(fin, f);
  if (st != CSA2_OK) return st;
  if (codes == nullptr || scales == nullptr || !aligned(codes, 4)) return CSA2_ERR_INVALID_ARG;
  if (fin->w_idx != nullptr) {
    if (idx_codes == nullptr || idx_scales == nullptr || !aligned(idx_codes, 8)) return CSA2_ERR_INVALID_ARG;
  } else if (idx_codes != nullptr || idx_scales != nullptr || k_f32 != nullptr) {
    return CSA2_ERR_INVALID_ARG;
  }
  if ((x_f32 && !aligned(x_f32, 16)) || (k_f32 && !aligned(k_f32, 16))) return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}
}  // namespace

csa2_status csa2_kv_finish_rows(const float *c, int64_t tokens, int32_t n_layers, int64_t pos0,
                                const csa2_kv_finish *fin, uint8_t *codes, uint8_t *scales, uint8_t *idx_codes,
                                uint8_t *idx_scales, float *x_f32, float *k_f32, csa2_stream stream) {
  CSA2_TRACE;
  KvFinish f;
  csa2_status st = check_finish_rows(tokens, n_layers, pos0, fin, codes, scales, idx_codes, idx_scales, x_f32,
                                     k_f32, &f);
  if (st != CSA2_OK) return st;
  if (tokens == 0 || n_layers == 0) return CSA2_OK;
  if (c == nullptr || !aligned(c, 16)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_kv_finish_rows(c, tokens, n_layers, pos0, f, codes, scales, idx_codes, idx_scales, x_f32,
                                        k_f32, as_stream(stream)));
}

csa2_status csa2_ced_kv_project_finished(const uint16_t *h, int64_t tokens, int32_t hidden, int32_t n_layers,
                                         const uint16_t *w_kv, const csa2_kv_finish *fin, int64_t pos0,
                                         float *c_f32, uint8_t *codes, uint8_t *scales, uint8_t *idx_codes,
                                         uint8_t *idx_scales, csa2_stream stream) {
  CSA2_TRACE;
  if (hidden <= 0 || hidden % 64 != 0 || tokens > (int64_t)1 << 31) return CSA2_ERR_INVALID_ARG;
  KvFinish f;
  csa2_status st = check_finish_rows(tokens, n_layers, pos0, fin, codes, scales, idx_codes, idx_scales, nullptr,
                                     nullptr, &f);
  if (st != CSA2_OK) return st;
  if (tokens == 0 || n_layers == 0) return CSA2_OK;
  if (h == nullptr || w_kv == nullptr || c_f32 == nullptr) return CSA2_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(w_kv, 16) || !aligned(c_f32, 16)) return CSA2_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_ced_project(h, tokens, hidden, n_layers, w_kv, nullptr, nullptr, nullptr, nullptr, c_f32, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(launch_kv_finish_rows(c_f32, tokens, n_layers, pos0, f, codes, scales, idx_codes, idx_scales,
                                        nullptr, nullptr, s));
}

csa2_status csa2_kv_append_finished(const csa2_kv_layer *layer, const csa2_seqs *seqs, const float *latent,
                                    const csa2_kv_finish *fin, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  KvFinish f;
  csa2_status st = check_layer(layer, true, false, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if ((st = check_finish(fin, &f)) != CSA2_OK) return st;
  if (L.rope_dim != 0 || !aligned(layer->codes, 4)) return CSA2_ERR_INVALID_ARG;
  const bool fp4_keys = layer->idx_keys != nullptr && layer->idx_dtype == CSA2_FP4;
  if (fp4_keys != (fin->w_idx != nullptr)) return CSA2_ERR_INVALID_ARG;
  if (fp4_keys && !keys_ok(layer)) return CSA2_ERR_INVALID_ARG;
  if (!fp4_keys && layer->idx_keys != nullptr) return CSA2_ERR_INVALID_ARG;
  if (S.batch == 0) return CSA2_OK;
  if (latent == nullptr || !aligned(latent, 16)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_kv_append_finish(L, S, latent, f, as_stream(stream)));
}

csa2_status csa2_swa_append(const csa2_swa_window *win, const int32_t *positions, int32_t batch,
                            const float *latent, csa2_stream stream) {
  CSA2_TRACE;
  if (win == nullptr || batch < 0 || batch > kMaxBatch || batch > win->batch) return CSA2_ERR_INVALID_ARG;
  if (batch == 0) return CSA2_OK;
  if (win->codes == nullptr || win->scales == nullptr || positions == nullptr || latent == nullptr)
    return CSA2_ERR_INVALID_ARG;
  if (!aligned(win->codes, 8) || !aligned(win->scales, 4) || !aligned(latent, 16)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_swa_append(win->codes, win->scales, positions, batch, latent, as_stream(stream)));
}

csa2_status csa2_swa_attn_merge(const csa2_swa_window *win, const int32_t *seq_lens, int32_t batch,
                                const uint16_t *q, int32_t heads, int32_t q_dim, float softmax_scale, float *out,
                                float *lse, csa2_stream stream) {
  CSA2_TRACE;
  if (win == nullptr || batch < 0 || batch > kMaxBatch || batch > win->batch) return CSA2_ERR_INVALID_ARG;
  if (heads < 16 || heads > 128 || heads % 16 != 0 || (q_dim != 512 && q_dim != 576)) return CSA2_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 3.0e38f)) return CSA2_ERR_INVALID_ARG;
  if (batch == 0) return CSA2_OK;
  if (win->codes == nullptr || win->scales == nullptr || seq_lens == nullptr || q == nullptr || out == nullptr ||
      lse == nullptr)
    return CSA2_ERR_INVALID_ARG;
  if (!aligned(win->codes, 16) || !aligned(q, 16) || !aligned(out, 4) || !aligned(lse, 4)) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_swa_attn_merge(win->codes, win->scales, seq_lens, batch, q, heads, q_dim, softmax_scale,
                                        out, lse, as_stream(stream)));
}

csa2_status csa2_ced_kv_project(const uint16_t *h, int64_t tokens, int32_t hidden, int32_t n_layers,
                                const uint16_t *w_kv, const uint16_t *w_z, uint8_t *codes, uint8_t *scales,
                                uint16_t *z, float *c_f32, csa2_stream stream) {
  CSA2_TRACE;
  if (tokens < 0 || n_layers < 0 || hidden <= 0 || hidden % 64 != 0) return CSA2_ERR_INVALID_ARG;
  if (tokens > (int64_t)1 << 31 || n_layers > 4096) return CSA2_ERR_INVALID_ARG;
  if (tokens == 0 || n_layers == 0) return CSA2_OK;
  if (h == nullptr || w_kv == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_INVALID_ARG;
  if ((z == nullptr) != (w_z == nullptr)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(w_kv, 16) || (w_z && !aligned(w_z, 16)) || !aligned(codes, 8) ||
      (z && !aligned(z, 16)) || (c_f32 && !aligned(c_f32, 16)))
    return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_ced_project(h, tokens, hidden, n_layers, w_kv, w_z, codes, scales, z, c_f32,
                                     as_stream(stream)));
}

csa2_status csa2_index_scores(const csa2_kv_layer *keys, const csa2_seqs *seqs, const void *q_idx,
                              const float *w_idx, float *scores, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(keys, false, true, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (S.batch == 0 || S.max_len == 0) return CSA2_OK;
  if (!query_ok(keys, q_idx, w_idx) || scores == nullptr) return CSA2_ERR_INVALID_ARG;
  return from_hip(launch_index_scores(L, S, IdxQuery{q_idx, w_idx}, scores, as_stream(stream)));
}

csa2_status csa2_topk_workspace_size(int32_t batch, int32_t max_len, int32_t top_k, size_t *bytes) {
  if (bytes == nullptr || batch < 0 || batch > kMaxBatch || max_len < 0 || max_len > kMaxSelectLen || top_k < 1 ||
      top_k > kMaxTopK)
    return CSA2_ERR_INVALID_ARG;
  *bytes = topk_workspace_bytes(batch, max_len, top_k);
  return CSA2_OK;
}

csa2_status csa2_topk(const float *scores, int64_t row_stride, const int32_t *lens, int32_t batch, int32_t max_len,
                      int32_t top_k, int32_t *indices, void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  if (batch < 0 || batch > kMaxBatch || max_len < 0 || max_len > kMaxSelectLen || top_k < 1 || top_k > kMaxTopK ||
      row_stride < max_len)
    return CSA2_ERR_INVALID_ARG;
  if (batch == 0) return CSA2_OK;
  if (scores == nullptr || lens == nullptr || indices == nullptr) return CSA2_ERR_INVALID_ARG;
  const size_t need = topk_workspace_bytes(batch, max_len, top_k);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  return from_hip(launch_topk_scores(scores, row_stride, lens, batch, max_len, top_k, indices, ws, as_stream(stream)));
}

csa2_status csa2_index_select_workspace_size(int32_t batch, int32_t max_seq_len, int32_t top_k, int32_t pool_blocks,
                                             int32_t pool_block_tokens, size_t *bytes) {
  if (bytes == nullptr || batch < 0 || batch > kMaxBatch || max_seq_len < 0 || max_seq_len > kMaxSelectLen ||
      top_k < 1 || top_k > kMaxTopK)
    return CSA2_ERR_INVALID_ARG;
  if (pool_blocks < 0 || pool_blocks > kMaxPoolBlocks) return CSA2_ERR_INVALID_ARG;
  if (pool_blocks > 0 && pool_block_tokens != 8) return CSA2_ERR_INVALID_ARG;
  *bytes = index_select_workspace_bytes(batch, max_seq_len, top_k, pool_blocks);
  return CSA2_OK;
}

csa2_status csa2_index_select(const csa2_kv_layer *keys, const csa2_seqs *seqs, const void *q_idx,
                              const float *w_idx, int32_t top_k, int32_t mode, const int32_t *pool_in,
                              int32_t *pool_out, int32_t pool_blocks,
                              int32_t pool_block_tokens, int32_t *indices, void *ws, size_t ws_bytes,
                              csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(keys, false, true, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX) return CSA2_ERR_INVALID_ARG;
  const bool pooled = (mode == CSA2_REINDEX) || pool_out != nullptr;
  if (pooled) {
    if (pool_block_tokens != 8 || pool_blocks < 1 || pool_blocks > kMaxPoolBlocks) return CSA2_ERR_INVALID_ARG;
  }
  if (mode == CSA2_REINDEX && (pool_in == nullptr || pool_out != nullptr)) return CSA2_ERR_INVALID_ARG;
  if (mode == CSA2_FULL && pool_in != nullptr) return CSA2_ERR_INVALID_ARG;
  if (S.batch == 0) return CSA2_OK;
  if (!query_ok(keys, q_idx, w_idx) || indices == nullptr) return CSA2_ERR_INVALID_ARG;
  const size_t need = index_select_workspace_bytes(S.batch, S.max_len, top_k, pooled ? pool_blocks : 0);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  hipError_t e;
  const IdxQuery q{q_idx, w_idx};
  if (mode == CSA2_FULL)
    e = launch_index_select_full(L, S, q, top_k, pool_out, pool_out ? pool_blocks : 0, indices, ws,
                                 as_stream(stream));
  else
    e = launch_index_select_reindex(L, S, q, top_k, pool_in, pool_blocks, indices, ws, as_stream(stream));
  return from_hip(e);
}

namespace {
// Validates one row of csa2_index_select_append (the checks of csa2_kv_append).
csa2_status check_append(const csa2_append &a, AppendRow *out) {
  KvLayerDev L;
  csa2_status st = check_layer(a.layer, a.latent != nullptr, false, &L);
  if (st != CSA2_OK) return st;
  if (a.latent == nullptr && a.rope == nullptr && a.idx_key == nullptr) return CSA2_ERR_INVALID_ARG;
  if (a.rope != nullptr && (L.rope_dim == 0 || a.layer->rope == nullptr)) return CSA2_ERR_INVALID_ARG;
  if (a.latent != nullptr && L.rope_dim != 0 && a.rope == nullptr) return CSA2_ERR_INVALID_ARG;
  if (a.idx_key != nullptr && !keys_ok(a.layer)) return CSA2_ERR_INVALID_ARG;
  if (a.idx_key != nullptr && !aligned(a.idx_key, 16)) return CSA2_ERR_INVALID_ARG;
  *out = AppendRow{L, a.latent, a.rope, a.idx_key};
  return CSA2_OK;
}
}  // namespace

csa2_status csa2_index_select_append(const csa2_kv_layer *keys, const csa2_seqs *seqs, const csa2_append *appends,
                                     int32_t n_appends, const void *q_idx, const float *w_idx, int32_t top_k,
                                     int32_t *pool_out, int32_t pool_blocks, int32_t pool_block_tokens,
                                     int32_t *indices, void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(keys, false, true, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (pool_out != nullptr && (pool_block_tokens != 8 || pool_blocks < 1 || pool_blocks > kMaxPoolBlocks))
    return CSA2_ERR_INVALID_ARG;
  if (n_appends < 0 || n_appends > kMaxAppendRows || (n_appends > 0 && appends == nullptr))
    return CSA2_ERR_INVALID_ARG;
  AppendRow rows[kMaxAppendRows];
  const void *new_key = nullptr;
  for (int i = 0; i < n_appends; ++i) {
    if ((st = check_append(appends[i], &rows[i])) != CSA2_OK) return st;
    // rows write disjoint storage: no two appends may share codes or key storage
    for (int j = 0; j < i; ++j) {
      if (appends[i].latent && appends[j].latent && appends[i].layer->codes == appends[j].layer->codes)
        return CSA2_ERR_INVALID_ARG;
      if (appends[i].idx_key && appends[j].idx_key && appends[i].layer->idx_keys == appends[j].layer->idx_keys)
        return CSA2_ERR_INVALID_ARG;
    }
    if (appends[i].idx_key != nullptr && appends[i].layer->idx_keys == keys->idx_keys) {
      const csa2_kv_layer *a = appends[i].layer;  // the scanned keys: the same kind of key
      if (a->idx_dtype != keys->idx_dtype || a->idx_scales != keys->idx_scales) return CSA2_ERR_INVALID_ARG;
      new_key = appends[i].idx_key;
    }
  }
  if (S.batch == 0) return CSA2_OK;
  if (!query_ok(keys, q_idx, w_idx) || indices == nullptr) return CSA2_ERR_INVALID_ARG;
  const size_t need = index_select_workspace_bytes(S.batch, S.max_len, top_k, pool_out ? pool_blocks : 0);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  return from_hip(launch_index_select_full(L, S, IdxQuery{q_idx, w_idx}, top_k, pool_out, pool_out ? pool_blocks : 0,
                                           indices, ws, as_stream(stream), rows, n_appends, new_key));
}

csa2_status csa2_index_reindex_layers_workspace_size(int32_t n_layers, int32_t batch, int32_t top_k,
                                                    int32_t pool_blocks, int32_t pool_block_tokens, size_t *bytes) {
  if (bytes == nullptr || n_layers < 1 || n_layers > kMaxIdxLayers || batch < 0 || batch > kMaxBatch || top_k < 1 ||
      top_k > kMaxTopK)
    return CSA2_ERR_INVALID_ARG;
  if (pool_block_tokens != 8 || pool_blocks < 1 || pool_blocks > kMaxPoolBlocks) return CSA2_ERR_INVALID_ARG;
  *bytes = reindex_layers_workspace_bytes(n_layers, batch);
  return CSA2_OK;
}

csa2_status csa2_index_reindex_layers(const csa2_kv_layer *keys, const csa2_seqs *seqs,
                                      const csa2_reindex_query *queries, int32_t n_layers, int32_t top_k,
                                      const int32_t *pool_in, int32_t pool_blocks, int32_t pool_block_tokens,
                                      void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(keys, false, true, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (queries == nullptr || n_layers < 1 || n_layers > kMaxIdxLayers) return CSA2_ERR_INVALID_ARG;
  if (top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (pool_block_tokens != 8 || pool_blocks < 1 || pool_blocks > kMaxPoolBlocks) return CSA2_ERR_INVALID_ARG;
  if (S.batch == 0) return CSA2_OK;
  if (pool_in == nullptr) return CSA2_ERR_INVALID_ARG;
  IdxQuery q[kMaxIdxLayers];
  int32_t *out[kMaxIdxLayers];
  for (int j = 0; j < n_layers; ++j) {
    if (!query_ok(keys, queries[j].q_idx, queries[j].w_idx) || queries[j].indices == nullptr)
      return CSA2_ERR_INVALID_ARG;
    q[j] = IdxQuery{queries[j].q_idx, queries[j].w_idx};
    out[j] = queries[j].indices;
  }
  const size_t need = reindex_layers_workspace_bytes(n_layers, S.batch);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  return from_hip(launch_reindex_layers(L, S, q, out, n_layers, top_k, pool_in, pool_blocks, ws, as_stream(stream)));
}

csa2_status csa2_attn_workspace_size(int32_t batch, int32_t heads, int32_t top_k, int32_t latent_dim, size_t *bytes) {
  if (bytes == nullptr || batch < 0 || batch > kMaxBatch || heads <= 0 || heads % 16 != 0 || heads > 128 ||
      top_k < 1 || top_k > kMaxTopK || latent_dim != 512)
    return CSA2_ERR_INVALID_ARG;
  *bytes = attn_workspace_bytes(1, batch, heads, top_k, false);
  return CSA2_OK;
}

csa2_status csa2_attn_swa_workspace_size(int32_t batch, int32_t heads, int32_t top_k, int32_t latent_dim,
                                         size_t *bytes) {
  if (bytes == nullptr || batch < 0 || batch > kMaxBatch || heads <= 0 || heads % 16 != 0 || heads > 128 ||
      top_k < 1 || top_k > kMaxTopK || latent_dim != 512)
    return CSA2_ERR_INVALID_ARG;
  *bytes = attn_workspace_bytes(1, batch, heads, top_k, true);
  return CSA2_OK;
}

csa2_status csa2_sparse_fp4_decode_attn(const csa2_kv_layer *layer, const csa2_seqs *seqs, const uint16_t *q,
                                        int32_t heads, const int32_t *indices, int32_t top_k, float softmax_scale,
                                        float *out, float *lse, void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(layer, true, false, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (heads <= 0 || heads % 16 != 0 || heads > 128 || top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 1e30f)) return CSA2_ERR_INVALID_ARG;
  if (S.batch == 0) return CSA2_OK;
  if (q == nullptr || indices == nullptr || out == nullptr || !aligned(q, 16) || !aligned(out, 16))
    return CSA2_ERR_INVALID_ARG;
  const size_t need = attn_workspace_bytes(1, S.batch, heads, top_k, false);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  const AttnLaunchJob job{L, q, indices, nullptr, nullptr, nullptr, out, lse};
  return from_hip(launch_sparse_attn(&job, 1, S, heads, top_k, softmax_scale, ws, ~(size_t)0, as_stream(stream)));
}

csa2_status csa2_sparse_fp4_decode_attn_swa(const csa2_kv_layer *layer, const csa2_seqs *seqs, const uint16_t *q,
                                            int32_t heads, const int32_t *indices, int32_t top_k,
                                            float softmax_scale, const csa2_swa_window *win, const float *new_latent,
                                            float *out, float *lse, void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  KvLayerDev L;
  SeqsDev S;
  csa2_status st = check_layer(layer, true, false, &L);
  if (st != CSA2_OK) return st;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if (heads <= 0 || heads % 16 != 0 || heads > 128 || top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 1e30f)) return CSA2_ERR_INVALID_ARG;
  if (win == nullptr || win->batch < S.batch) return CSA2_ERR_INVALID_ARG;
  if (S.batch == 0) return CSA2_OK;
  if (q == nullptr || indices == nullptr || out == nullptr || !aligned(q, 16) || !aligned(out, 16))
    return CSA2_ERR_INVALID_ARG;
  if (win->codes == nullptr || win->scales == nullptr || !aligned(win->codes, 16) || !aligned(win->scales, 4))
    return CSA2_ERR_INVALID_ARG;
  if (new_latent != nullptr && !aligned(new_latent, 8)) return CSA2_ERR_INVALID_ARG;
  const size_t need = attn_workspace_bytes(1, S.batch, heads, top_k, true);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  const AttnLaunchJob job{L, q, indices, win->codes, win->scales, new_latent, out, lse};
  return from_hip(launch_sparse_attn(&job, 1, S, heads, top_k, softmax_scale, ws, ~(size_t)0, as_stream(stream)));
}

csa2_status csa2_attn_layers_workspace_size(int32_t n_layers, int32_t batch, int32_t heads, int32_t top_k,
                                            int32_t latent_dim, int32_t with_window, size_t *bytes) {
  if (bytes == nullptr || n_layers < 1 || n_layers > kMaxAttnJobs || batch < 0 ||
      (int64_t)n_layers * batch > kMaxBatch || heads <= 0 || heads % 16 != 0 || heads > 128 || top_k < 1 ||
      top_k > kMaxTopK || latent_dim != 512)
    return CSA2_ERR_INVALID_ARG;
  *bytes = attn_workspace_bytes(n_layers, batch, heads, top_k, with_window != 0);
  return CSA2_OK;
}

namespace {
// The layered attention with its partials bounded by max_ws bytes (the split
// count lowered to fit): the workspace entry point passes no bound, the
// allocation-free one its scratch size.
csa2_status attn_layers_impl(const csa2_attn_layer *layers, int32_t n_layers, const csa2_seqs *seqs, int32_t heads,
                             int32_t top_k, float softmax_scale, void *ws, size_t ws_bytes, size_t max_ws,
                             csa2_stream stream) {
  SeqsDev S;
  csa2_status st;
  if (layers == nullptr || n_layers < 1 || n_layers > kMaxAttnJobs) return CSA2_ERR_INVALID_ARG;
  if ((st = check_seqs(seqs, &S)) != CSA2_OK) return st;
  if ((int64_t)n_layers * S.batch > kMaxBatch) return CSA2_ERR_INVALID_ARG;
  if (heads <= 0 || heads % 16 != 0 || heads > 128 || top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 1e30f)) return CSA2_ERR_INVALID_ARG;
  AttnLaunchJob jobs[kMaxAttnJobs];
  const bool window = layers[0].win != nullptr;
  for (int j = 0; j < n_layers; ++j) {
    const csa2_attn_layer &x = layers[j];
    KvLayerDev L;
    if ((st = check_layer(x.layer, true, false, &L)) != CSA2_OK) return st;
    if (j > 0 && L.rope_dim != jobs[0].L.rope_dim) return CSA2_ERR_INVALID_ARG;  // one kernel variant per launch
    if ((x.win != nullptr) != window) return CSA2_ERR_INVALID_ARG;
    if (x.win == nullptr && x.new_latent != nullptr) return CSA2_ERR_INVALID_ARG;
    if (x.win != nullptr) {
      if (x.win->batch < S.batch) return CSA2_ERR_INVALID_ARG;
      if (S.batch > 0 && (x.win->codes == nullptr || x.win->scales == nullptr || !aligned(x.win->codes, 16) ||
                          !aligned(x.win->scales, 4)))
        return CSA2_ERR_INVALID_ARG;
      if (x.new_latent != nullptr && !aligned(x.new_latent, 8)) return CSA2_ERR_INVALID_ARG;
    }
    if (S.batch > 0 && (x.q == nullptr || x.indices == nullptr || x.out == nullptr || !aligned(x.q, 16) ||
                        !aligned(x.out, 16)))
      return CSA2_ERR_INVALID_ARG;
    jobs[j] = AttnLaunchJob{L,
                            x.q,
                            x.indices,
                            x.win ? x.win->codes : nullptr,
                            x.win ? x.win->scales : nullptr,
                            x.new_latent,
                            x.out,
                            x.lse};
  }
  if (S.batch == 0) return CSA2_OK;
  const size_t need = attn_workspace_bytes(n_layers, S.batch, heads, top_k, window, max_ws);
  if (ws == nullptr || ws_bytes < need || need > max_ws || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  return from_hip(launch_sparse_attn(jobs, n_layers, S, heads, top_k, softmax_scale, ws, max_ws, as_stream(stream)));
}
}  // namespace

csa2_status csa2_sparse_fp4_decode_attn_layers(const csa2_attn_layer *layers, int32_t n_layers,
                                               const csa2_seqs *seqs, int32_t heads, int32_t top_k,
                                               float softmax_scale, void *ws, size_t ws_bytes, csa2_stream stream) {
  CSA2_TRACE;
  return attn_layers_impl(layers, n_layers, seqs, heads, top_k, softmax_scale, ws, ws_bytes, ~(size_t)0, stream);
}

csa2_status csa2_sparse_fp4_decode_attn_layers_noalloc(const csa2_attn_layer *layers, int32_t n_layers,
                                                       const csa2_seqs *seqs, int32_t heads, int32_t top_k,
                                                       float softmax_scale, csa2_stream stream) {
  CSA2_TRACE;
  SeqsDev S;
  csa2_status st = check_seqs(seqs, &S);
  if (st != CSA2_OK) return st;
  if (layers == nullptr || n_layers < 1 || n_layers > kMaxAttnJobs) return CSA2_ERR_INVALID_ARG;
  if ((int64_t)n_layers * S.batch > kMaxBatch) return CSA2_ERR_INVALID_ARG;
  if (heads <= 0 || heads % 16 != 0 || heads > 128 || top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_INVALID_ARG;
  const bool window = layers[0].win != nullptr;
  if (attn_workspace_bytes(n_layers, S.batch, heads, top_k, window, kAttnScratchBytes) > kAttnScratchBytes)
    return CSA2_ERR_WORKSPACE;
  void *scratch_ptr = nullptr;
  if (attn_scratch(&scratch_ptr) != hipSuccess) return CSA2_ERR_HIP;
  return attn_layers_impl(layers, n_layers, seqs, heads, top_k, softmax_scale, scratch_ptr, kAttnScratchBytes,
                          kAttnScratchBytes, stream);
}

csa2_block_pool *csa2_block_pool_create(int32_t num_blocks) {
  if (num_blocks < 0) return nullptr;
  csa2_block_pool *p = new (std::nothrow) csa2_block_pool;
  if (p == nullptr) return nullptr;
  try {
    p->free_ids.resize(num_blocks);
    p->is_free.assign(num_blocks, 1);
  } catch (...) {
    delete p;
    return nullptr;
  }
  // pop order: lowest id first
  for (int32_t i = 0; i < num_blocks; ++i) p->free_ids[i] = num_blocks - 1 - i;
  return p;
}

csa2_status csa2_block_alloc(csa2_block_pool *pool, int32_t n, int32_t *ids_out) {
  if (pool == nullptr || n < 0 || (n > 0 && ids_out == nullptr)) return CSA2_ERR_INVALID_ARG;
  if ((size_t)n > pool->free_ids.size()) return CSA2_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = pool->free_ids.back();
    pool->free_ids.pop_back();
    pool->is_free[id] = 0;
    ids_out[i] = id;
  }
  return CSA2_OK;
}

csa2_status csa2_block_free(csa2_block_pool *pool, int32_t n, const int32_t *ids) {
  if (pool == nullptr || n < 0 || (n > 0 && ids == nullptr)) return CSA2_ERR_INVALID_ARG;
  const int32_t nb = (int32_t)pool->is_free.size();
  // validate everything first (no partial frees), including duplicates within ids
  std::vector<uint8_t> seen;
  try {
    seen.assign(nb, 0);
  } catch (...) {
    return CSA2_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= nb || pool->is_free[id] || seen[id]) return CSA2_ERR_INVALID_ARG;
    seen[id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->is_free[ids[i]] = 1;
    pool->free_ids.push_back(ids[i]);
  }
  return CSA2_OK;
}

int32_t csa2_block_pool_num_free(const csa2_block_pool *pool) {
  return pool == nullptr ? -1 : (int32_t)pool->free_ids.size();
}

void csa2_block_pool_destroy(csa2_block_pool *pool) { delete pool; }

}  // extern "C"
