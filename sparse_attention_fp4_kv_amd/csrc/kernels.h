// Internal launch interface between the C ABI layer (api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/csa2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Kernels that csa2_time_next_launch can time (names in api.hip).
enum KernelId {
  kKernIndexScan = 0,   // full scan of the indexer keys (per-position or block-max keys)
  kKernPoolScore,       // scoring of the pool positions (Reindex, and the Full layer's own top-K)
  kKernTopkGiven,       // key conversion of caller-given scores
  kKernTopkCompact,     // threshold compaction + exact refine
  kKernSparseAttn,
  kKernAttnCombine,
  kKernCedProject,
  kKernFp4Pack,
  kKernKvAppend,
  kKernIndexScores,
  kKernKvFinish,
  kKernSwaAttn,
  kKernCount
};
// Records the armed event pair around the next launch of `id` (no-op otherwise).
void timer_before(KernelId id, hipStream_t st);
void timer_after(KernelId id, hipStream_t st);

// Debug checks: while they are on, kernels OR these bits (the public
// CSA2_DBG_* values) into a per-device flag word; debug_flags() is that
// word's device address on the current device, or null when the checks are
// off (then every check is skipped).
constexpr uint32_t kDbgQRange = 1u, kDbgIndex = 2u, kDbgPage = 4u, kDbgNonFinite = 8u, kDbgScore = 16u,
                   kDbgSeqLen = 32u;
constexpr int kMaxDevices = 64;  // devices whose per-device library state is kept
uint32_t *debug_flags();
__device__ __forceinline__ void dbg_raise(uint32_t *dbg, uint32_t bit) {
  if (dbg != nullptr) atomicOr(dbg, bit);
}

// Device view of one KV layer's paged pool (validated copy of csa2_kv_layer).
struct KvLayerDev {
  uint8_t *codes;
  uint8_t *scales;
  uint16_t *rope;
  void *idx_keys;
  uint8_t *idx_scales;  // FP4 keys
  int num_blocks;
  int rope_dim;   // 0 or 64
  int idx_f32;    // 1: fp32 keys (64 dims)
  int idx_fp4;    // 1: FP4 keys (128 dims, multi-head score); else bf16 (64 dims)
  int idx_heads;  // query heads of the FP4 score (1 .. 32)
};

// The indexer query of one call: fp32 [B][64] for fp32 / bf16 keys (w null),
// fp16 [B][idx_heads][128] plus fp32 weights [B][idx_heads] for FP4 keys.
struct IdxQuery {
  const void *q;
  const float *w;
};

// Device view of a batch (validated copy of csa2_seqs).
struct SeqsDev {
  const int32_t *block_table;
  const int32_t *seq_lens;
  int max_blocks;
  int batch;
  int max_len;  // host bound of seq_lens
};

hipError_t launch_fp4_pack(const float *x, int64_t rows, int channels, uint8_t *codes, uint8_t *scales,
                           hipStream_t st);
hipError_t launch_fp4_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int channels, float *y,
                             hipStream_t st);
hipError_t launch_kv_append(const KvLayerDev &L, const SeqsDev &S, const float *latent, const uint16_t *rope,
                            const void *idx_key, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);

// ---- indexer / top-K (indexer.hip)
size_t topk_workspace_bytes(int batch, int max_items, int top_k);
hipError_t launch_index_scores(const KvLayerDev &L, const SeqsDev &S, IdxQuery q, float *scores, hipStream_t st);
hipError_t launch_topk_scores(const float *scores, int64_t stride, const int32_t *lens, int batch, int max_len,
                              int top_k, int32_t *indices, void *ws, hipStream_t st);
size_t index_select_workspace_bytes(int batch, int max_len, int top_k, int pool_blocks);
// A row appended at position seq_lens[b] - 1 of every sequence in the same
// launch as a Full-mode scan (the append workgroups ride along).
constexpr int kMaxAppendRows = 8;
struct AppendRow {
  KvLayerDev L;
  const float *latent;
  const uint16_t *rope;
  const void *idx_key;
};
// new_key: the key input of the append that writes the scanned keys (scored
// from there), or null.
hipError_t launch_index_select_full(const KvLayerDev &L, const SeqsDev &S, IdxQuery q_idx, int top_k,
                                    int32_t *pool_out, int pool_blocks, int32_t *indices, void *ws,
                                    hipStream_t st, const AppendRow *app = nullptr, int n_app = 0,
                                    const void *new_key = nullptr);
hipError_t launch_index_select_reindex(const KvLayerDev &L, const SeqsDev &S, IdxQuery q_idx, int top_k,
                                       const int32_t *pool_in, int pool_blocks, int32_t *indices, void *ws,
                                       hipStream_t st);
// Reindex of several layers (own query and output each) over one key pool and
// one candidate pool: two launches in all.  At most kMaxIdxLayers layers.
constexpr int kMaxIdxLayers = 8;
size_t reindex_layers_workspace_bytes(int jobs, int batch);
hipError_t launch_reindex_layers(const KvLayerDev &L, const SeqsDev &S, const IdxQuery *q_idx, int32_t *const *indices,
                                 int jobs, int top_k, const int32_t *pool_in, int pool_blocks, void *ws,
                                 hipStream_t st);

// ---- attention (attention.hip)
// One launch serves up to kMaxAttnJobs attention problems over one batch view
// (e.g. the layers of a step, each with its own KV pool, query, indices and
// output).  window: the sliding-window ring's codes / scales join the softmax
// as four more splits (all jobs of a launch have a window, or none);
// win_latent, if given, is the current token's window entry, appended to the
// ring in the same launch.
constexpr int kMaxAttnJobs = 20;
struct AttnLaunchJob {
  KvLayerDev L;
  const uint16_t *q;
  const int32_t *indices;
  uint8_t *win_codes;
  float *win_scales;
  const float *win_latent;
  float *out;
  float *lse;
};
// Workspace of an attention launch; max_bytes bounds the split partials (the
// split count is lowered to fit when it can be).
size_t attn_workspace_bytes(int jobs, int batch, int heads, int top_k, bool window,
                            size_t max_bytes = ~(size_t)0);
// The library-held scratch of the allocation-free entry point (device memory
// of this many bytes on every device it runs on) and its address on the
// current device.
constexpr size_t kAttnScratchBytes = (size_t)32 << 20;
hipError_t attn_scratch(void **ptr);

hipError_t launch_sparse_attn(const AttnLaunchJob *jobs, int n_jobs, const SeqsDev &S, int heads, int top_k,
                              float scale, void *ws, size_t max_ws, hipStream_t st);

// ---- CED projection (ced.hip)
// Latent finish (RMSNorm, RoPE, FP4 pack) and the FP4 indexer key projected
// from the cached entry.
struct KvFinish {
  const float *gamma;      // [layers][512]
  float eps;               // > 0
  float theta;             // RoPE base, 0: no rotation
  const uint16_t *w_idx;   // [layers][128][512] bf16, or null
};
hipError_t launch_kv_finish_rows(const float *c, int64_t tokens, int n_layers, int64_t pos0, const KvFinish &fin,
                                 uint8_t *codes, uint8_t *scales, uint8_t *k_codes, uint8_t *k_scales, float *x_f32,
                                 float *k_f32, hipStream_t st);
hipError_t launch_kv_append_finish(const KvLayerDev &L, const SeqsDev &S, const float *latent, const KvFinish &fin,
                                   hipStream_t st);

// Sliding-window branch: FP8 ring of 128 slots per sequence.
hipError_t launch_swa_append(uint8_t *codes, float *scales, const int32_t *pos, int batch, const float *latent,
                             hipStream_t st);
hipError_t launch_swa_attn_merge(const uint8_t *codes, const float *scales, const int32_t *lens, int batch,
                                 const uint16_t *q, int heads, int qdim, float softmax_scale, float *out, float *lse,
                                 hipStream_t st);

hipError_t launch_ced_project(const uint16_t *h, int64_t tokens, int hidden, int n_layers, const uint16_t *w_kv,
                              const uint16_t *w_z, uint8_t *codes, uint8_t *scales, uint16_t *z, float *c_f32,
                              hipStream_t st);

}  // namespace csa2
