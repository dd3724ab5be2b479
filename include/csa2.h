/*
 * csa2.h -- C ABI of libcsa2, the MI355X (gfx950) sparse FP4-KV decode path.
 *
 * The library implements, as hand-written HIP kernels, the hot path of the
 * DeepSeek-V4.1-Flash global KV cache described on these web pages:
 *   [P1] discuss.pytorch.kr, "DeepSeek-V4.1-Flash, KV cache 890 bytes per token"
 *        (sections "Causal Encoder-Decoder", "CSA2", "Hierarchical Sparse
 *        Indexer", "FP4 KV cache", "why the KV cache became the bottleneck")
 *   [P3] llmfeed.kr news summary, section "scale and structure"
 *   [P4] ingu627.github.io asymmetric-serving blog, sections 2 and 3
 *
 * Conventions (every entry point):
 *   - Pointers marked "device" are device memory owned by the caller.  The
 *     library never allocates device memory and keeps no pointer after a call
 *     returns.  Scratch memory comes in through a caller-owned workspace whose
 *     size the matching *_workspace_size call reports.
 *   - A workspace must be all zero before its first use (csa2_workspace_clear
 *     does that).  Every call leaves the parts it used zero again, so one
 *     workspace can serve a sequence of calls on one stream.  Calls that
 *     overlap in time on one workspace race; give concurrent streams their
 *     own workspaces.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  Host-side argument validation happens before any
 *     launch; a rejected call launches nothing and returns a status.
 *   - Launch failures return CSA2_ERR_HIP.  No exception crosses the ABI.
 *   - A call serves at most 65,535 sequences (csa2_seqs.batch and every
 *     `batch` argument, workspace-size calls included); more return
 *     CSA2_ERR_INVALID_ARG.
 *   - Device data is trusted only as far as stated: selected indices that are
 *     negative or >= the sequence length, and page ids outside
 *     [0, num_blocks), are skipped rather than read.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 6

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1,  /* null pointer, bad size or unsupported combination */
  CSA2_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement      */
  CSA2_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required        */
  CSA2_ERR_HIP = 4           /* a HIP launch or runtime call failed               */
} csa2_status;

/* Indexer key storage.  CSA2_FP4: the latent's FP4 format applied to the
 * keys ([P1] "FP4 KV cache"), for the multi-head indexer of [P1] "CSA2". */
typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1, CSA2_FP4 = 2 } csa2_dtype;

/* CSA2 layer modes that run the indexer ([P1] "CSA2", mode table).  Reuse
 * mode runs no indexer: pass an earlier call's indices to the attention of
 * another layer. */
typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1 } csa2_mode;

typedef void *csa2_stream; /* hipStream_t */

/* One KV layer's paged pool (structure of arrays, all device, caller-owned).
 * Token slot r = block * block_tokens + slot holds:
 *   codes   [num_blocks * block_tokens][latent_dim / 2]  E2M1 nibbles, byte j =
 *           channel 2j (low nibble) | channel 2j+1 (high nibble)
 *   scales  [num_blocks * block_tokens][latent_dim / 16] E4M3FN, one per 16 channels
 *   rope    [num_blocks * block_tokens][rope_dim] bf16, or NULL when rope_dim == 0
 *   idx_keys[num_blocks * block_tokens][idx_dim] of idx_dtype, or NULL for a
 *           layer that never selects; with CSA2_FP4 the E2M1 nibbles
 *           [..][idx_dim / 2] (byte j = dims 2j | 2j+1 << 4) and
 *   idx_scales[num_blocks * block_tokens][idx_dim / 16] E4M3FN, one per 16 dims
 * block_tokens must be 64; latent_dim must be 512; rope_dim 0 or 64.  Indexer:
 * CSA2_F32 / CSA2_BF16 keys have idx_dim 64 and idx_heads 1 (one query);
 * CSA2_FP4 keys have idx_dim 128 and idx_heads in [1, 32] query heads
 * ([P1] "CSA2": 32 indexer query heads of dimension 128). */
typedef struct {
  uint8_t *codes;
  uint8_t *scales;
  uint16_t *rope;
  void *idx_keys;
  int32_t num_blocks;
  int32_t block_tokens;
  int32_t latent_dim;
  int32_t rope_dim;
  int32_t idx_dim;
  int32_t idx_dtype;   /* csa2_dtype */
  uint8_t *idx_scales; /* CSA2_FP4 keys only, else NULL */
  int32_t idx_heads;
} csa2_kv_layer;

/* Batch view.  Position p of sequence b lives in slot
 * block_table[b * max_blocks_per_seq + p / 64] * 64 + p % 64. */
typedef struct {
  const int32_t *block_table; /* device [batch][max_blocks_per_seq]                 */
  int32_t max_blocks_per_seq;
  const int32_t *seq_lens;    /* device [batch]: visible tokens of each sequence     */
  int32_t batch;              /* 0 .. 65,535 sequences per call (one grid
                                 dimension spans them)                              */
  int32_t max_seq_len;        /* host upper bound of seq_lens (sizes the launches);
                                 0 means max_blocks_per_seq * 64                      */
} csa2_seqs;

int csa2_abi_version(void);
const char *csa2_status_string(csa2_status status);

/* Profiling aid (not for concurrent use from several host threads): arms a
 * one-shot timer on the next launch of the named kernel -- hipEventRecord of
 * start_event (a hipEvent_t) just before it and of stop_event just after it,
 * on the stream it is launched on.  Names: "index_scan" (the Full-mode key
 * scan), "pool_score", "topk_given", "topk_compact", "sparse_attn",
 * "attn_combine", "ced_project", "fp4_pack", "kv_append", "index_scores".
 * kernel == NULL disarms.  Returns CSA2_ERR_INVALID_ARG for an unknown name. */
csa2_status csa2_time_next_launch(const char *kernel, void *start_event, void *stop_event);
/* 1 while a timer armed by csa2_time_next_launch has not fired yet (its kernel
 * has not been launched since), else 0. */
int32_t csa2_timer_pending(void);

/* ---- Debug checks: device-side checks of the documented input contracts.
 * Off unless the environment variable CSA2_DEBUG_CHECKS is a non-zero number
 * when the library first launches, or csa2_debug_checks(1) is called (0 turns
 * them off).  While on, kernels OR these bits into a per-device flag word
 * (inputs are still treated as documented: skipped entries stay skipped):
 *   CSA2_DBG_Q_RANGE    an attention query or rope value of magnitude above
 *                       65504 (fp16 overflow) or NaN
 *   CSA2_DBG_INDEX      a selected index below -1 or at or past seq_len
 *   CSA2_DBG_PAGE       a visible position whose page id is outside
 *                       [0, num_blocks) or past max_blocks_per_seq
 *   CSA2_DBG_NONFINITE  a NaN or infinite value given to the FP4 pack or append
 *   CSA2_DBG_SCORE      a NaN or infinite score given to csa2_topk
 *   CSA2_DBG_SEQ_LEN    a sequence length outside [0, max_seq_len]
 * csa2_debug_flags waits for the device, returns the bits raised on the
 * current device since the last call and clears them. */
#define CSA2_DBG_Q_RANGE 1u
#define CSA2_DBG_INDEX 2u
#define CSA2_DBG_PAGE 4u
#define CSA2_DBG_NONFINITE 8u
#define CSA2_DBG_SCORE 16u
#define CSA2_DBG_SEQ_LEN 32u
csa2_status csa2_debug_checks(int32_t enable);
csa2_status csa2_debug_flags(uint32_t *flags);

/* Zero `bytes` of a workspace on `stream` (a fill kernel, no memset node). */
csa2_status csa2_workspace_clear(void *ws, size_t bytes, csa2_stream stream);

/* ---- FP4 format ([P1] "FP4 KV cache": E2M1 elements, one E4M3 scale per 16
 * channels, no global scale).  For each row and 16-channel group g:
 *   s_g = E4M3(fl32(amax_g / 6)) rounded to nearest even, saturating at 448;
 *   element = nearest E2M1 grid point to |x| / s_g (ties to the even code,
 *   saturating at 6) with the sign of x; s_g == 0 zeroes the group.
 * x: device fp32 [rows][channels]; codes: device [rows][channels/2];
 * scales: device [rows][channels/16].  channels must be a positive multiple
 * of 16; rows >= 0 (0 is a no-op).  Bit-exact and deterministic. */
csa2_status csa2_fp4_pack(const float *x, int64_t rows, int32_t channels, uint8_t *codes,
                          uint8_t *scales, csa2_stream stream);

/* Inverse of the pack: y[r][c] = E2M1(nibble) * E4M3(scale) (exact in fp32). */
csa2_status csa2_fp4_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int32_t channels, float *y, csa2_stream stream);

/* ---- Decode-time append ([P1] "FP4 KV cache" format; the paged layout is
 * this library's).  For every sequence b, packs latent[b] (device fp32
 * [batch][latent_dim]) into the slot of position seq_lens[b] and copies
 * rope[b] (device bf16 [batch][rope_dim]) and idx_key[b] (device
 * [batch][idx_dim] of idx_dtype; fp32 for CSA2_FP4 keys, which are packed
 * like the latent) beside it.  Any of the three may be NULL
 * (not all): a key-only pool appends just idx_key; a layer with a rope
 * side-band needs rope whenever latent is given.  The caller increments
 * seq_lens afterwards.  A position whose page is not mapped (page index beyond
 * max_blocks_per_seq or page id outside the pool) is skipped. */
csa2_status csa2_kv_append(const csa2_kv_layer *layer, const csa2_seqs *seqs, const float *latent,
                           const uint16_t *rope, const void *idx_key, csa2_stream stream);

/* ---- CED projection with fused pack ([P1] "Causal Encoder-Decoder":
 * C_l = H W_l^KV, Z_l = H W_l^Z for every decoder layer l).
 *   h:     device bf16 [tokens][hidden]
 *   w_kv:  device bf16 [n_layers][512][hidden]  (out x in, W_l^KV transposed)
 *   w_z:   device bf16 [n_layers][64][hidden] or NULL
 *   codes: device [n_layers][tokens][256], scales: device [n_layers][tokens][32]
 *          (C_l packed from its fp32 accumulators exactly as csa2_fp4_pack)
 *   z:     device bf16 [n_layers][tokens][64] (round to nearest even) or NULL
 *   c_f32: device fp32 [n_layers][tokens][512] copy of the accumulators, or NULL
 * hidden must be a positive multiple of 64; tokens >= 0. */
csa2_status csa2_ced_kv_project(const uint16_t *h, int64_t tokens, int32_t hidden, int32_t n_layers,
                                const uint16_t *w_kv, const uint16_t *w_z, uint8_t *codes,
                                uint8_t *scales, uint16_t *z, float *c_f32, csa2_stream stream);

/* ---- Finishing a KV latent before it is cached, and the indexer key taken
 * from the cached entry.  [P1] "FP4 KV cache": the 512-channel latent is
 * RMS-normalised (learned weight) and rotated by RoPE before the FP4 pack;
 * [P1] "CSA2": a Full layer's indexer K is a projection of the main KV (32
 * indexer heads of dimension 128) and V4 keeps indexer keys in FP4.  This
 * library's reading of what the pages leave open, for a raw latent x at token
 * position p:
 *   y_j = x_j / sqrt(mean_j x_j^2 + eps) * gamma_j            (j < 512)
 *   channels 448 + 2i, 449 + 2i (i < 32) turned by the fp32 angle
 *   fl32(p * fl32(theta^(-2i/64))): (a, b) -> (a cos - b sin, a sin + b cos)
 *   entry = FP4 pack of y (csa2_fp4_pack rules)
 *   key   = FP4 pack of W_idx * dequant(entry)  (128 dims; 64 code bytes +
 *           8 scales, the CSA2_FP4 indexer-key layout)
 * fp32 arithmetic; p is taken exactly below 2^24. */
typedef struct {
  const float *gamma;     /* device fp32 [n_layers][512] RMSNorm weights */
  float eps;              /* RMSNorm epsilon, > 0 */
  float rope_theta;       /* RoPE base, > 0, or 0 for no rotation */
  const uint16_t *w_idx;  /* device bf16 [n_layers][128][512] (out x in), or NULL: no key */
} csa2_kv_finish;

/* Finishes rows c[l][t] (device fp32 [n_layers][tokens][512], position
 * pos0 + t, layer l's gamma and W_idx) into codes [n_layers][tokens][256] and
 * scales [..][32], and, with fin->w_idx, idx_codes [..][64] and idx_scales
 * [..][8].  x_f32 [..][512] (finished latent before packing) and k_f32
 * [..][128] (key before packing) are optional fp32 copies (NULL: skipped).
 * tokens, n_layers >= 0; pos0 >= 0 and pos0 + tokens <= 2^24. */
csa2_status csa2_kv_finish_rows(const float *c, int64_t tokens, int32_t n_layers, int64_t pos0,
                                const csa2_kv_finish *fin, uint8_t *codes, uint8_t *scales,
                                uint8_t *idx_codes, uint8_t *idx_scales, float *x_f32, float *k_f32,
                                csa2_stream stream);

/* csa2_ced_kv_project with the finish: C_l = H W_l^KV (fp32 accumulators,
 * written to c_f32 [n_layers][tokens][512], required: it is the hand-over
 * buffer) and then csa2_kv_finish_rows on C (token t at position pos0 + t).
 * No Z: the indexer key comes from the main KV. */
csa2_status csa2_ced_kv_project_finished(const uint16_t *h, int64_t tokens, int32_t hidden, int32_t n_layers,
                                         const uint16_t *w_kv, const csa2_kv_finish *fin, int64_t pos0,
                                         float *c_f32, uint8_t *codes, uint8_t *scales, uint8_t *idx_codes,
                                         uint8_t *idx_scales, csa2_stream stream);

/* csa2_kv_append with the finish: for every sequence b the raw latent[b]
 * (device fp32 [batch][512]) at position p = seq_lens[b] is finished and
 * stored in p's slot; with fin->w_idx (gamma [512], w_idx [128][512] of this
 * layer) its FP4 indexer key is stored beside it.  The layer has no rope
 * side-band (the rotation lives inside the latent); it has CSA2_FP4 indexer
 * keys exactly when fin->w_idx is given.  Unmapped pages are skipped. */
csa2_status csa2_kv_append_finished(const csa2_kv_layer *layer, const csa2_seqs *seqs, const float *latent,
                                    const csa2_kv_finish *fin, csa2_stream stream);

/* ---- The sliding-window branch.  [P1] "KV bottleneck": a local
 * sliding-window attention branch runs beside the global one; [P1] "Causal
 * Encoder-Decoder": the window n_win is 128; [P1] "FP4 KV cache": the SWA KV
 * stays in FP8.  This library's reading: a window entry is the layer's
 * 512-channel local latent (key = value, no rope part), stored as E4M3FN
 * codes with one fp32 scale per token (s = amax / 448, code =
 * E4M3_RNE(x / s) with x's sign, saturating); position p lives in ring slot
 * p mod 128; the window of a sequence of n positions is n-128 .. n-1; the two
 * branches form one softmax over the union of their entries. */
typedef struct {
  uint8_t *codes;  /* device [batch][128][512] E4M3FN, caller-owned */
  float *scales;   /* device [batch][128] */
  int32_t batch;   /* sequences the ring arrays hold */
} csa2_swa_window;

/* Packs latent[b] (device fp32 [batch][512]) into slot positions[b] mod 128
 * of sequence b's ring (positions: device int32 [batch], the new token's
 * position; negative: skipped).  batch <= win->batch. */
csa2_status csa2_swa_append(const csa2_swa_window *win, const int32_t *positions, int32_t batch,
                            const float *latent, csa2_stream stream);

/* Attention of every head over the window of each sequence (seq_lens: device
 * int32 [batch], positions held, current token included), merged in place
 * into the global branch's result: out (device fp32 [batch][heads][512]) and
 * lse (device fp32 [batch][heads], natural log; -inf for an empty global
 * selection) become the attention over the union of both branches' entries.
 * q: device bf16 [batch][heads][q_dim] (q_dim 512, or 576 with a rope part
 * that the window does not use); softmax_scale as for the global branch;
 * heads a multiple of 16 in [16, 128].  A sequence with an empty window is
 * left as it is. */
csa2_status csa2_swa_attn_merge(const csa2_swa_window *win, const int32_t *seq_lens, int32_t batch,
                                const uint16_t *q, int32_t heads, int32_t q_dim, float softmax_scale, float *out,
                                float *lse, csa2_stream stream);

/* ---- Indexer scores alone (the scoring step of [P1] "CSA2").  For
 * t < seq_lens[b], with k = the stored key of position t:
 *   CSA2_F32 / CSA2_BF16 keys: scores[b][t] = sum_d q_idx[b][d] * k[d],
 *     q_idx device fp32 [batch][idx_dim], w_idx NULL;
 *   CSA2_FP4 keys: scores[b][t] = sum_h w_idx[b][h] * max(0, sum_d q_idx[b][h][d] * k[d]),
 *     q_idx device fp16 [batch][idx_heads][idx_dim], w_idx device fp32
 *     [batch][idx_heads] (the combining rule across heads is this library's
 *     reading; the pages give only the head count and dimension).
 * fp32 accumulation; entries t >= seq_lens[b] up to max_seq_len are written
 * as -inf.  scores: device fp32 [batch][max_seq_len]. */
csa2_status csa2_index_scores(const csa2_kv_layer *keys, const csa2_seqs *seqs, const void *q_idx,
                              const float *w_idx, float *scores, csa2_stream stream);

/* ---- Top-K of given scores: for each row b the top_k largest of
 * scores[b][0 .. lens[b]) (ties: lower position wins), written to
 * indices[b][0..top_k) in increasing position order and padded with -1 when
 * lens[b] < top_k.  scores: device fp32 [batch][row_stride], finite;
 * lens: device int32 [batch]; max_len: host bound of lens (<= row_stride,
 * at most 8,388,608). */
csa2_status csa2_topk_workspace_size(int32_t batch, int32_t max_len, int32_t top_k, size_t *bytes);
csa2_status csa2_topk(const float *scores, int64_t row_stride, const int32_t *lens, int32_t batch,
                      int32_t max_len, int32_t top_k, int32_t *indices, void *ws, size_t ws_bytes,
                      csa2_stream stream);

/* ---- Index selection ([P1] "CSA2" Full / Reindex modes and "Hierarchical
 * Sparse Indexer").
 * FULL: scores every visible position of each sequence with q_idx[b] and
 *   writes the top_k positions to indices[b] (ascending, -1 padded).  When
 *   pool_out is not NULL it also gives each aligned run of pool_block_tokens
 *   positions the maximum score inside it and writes the ids of the best
 *   pool_blocks runs (ties: lower id) to pool_out[b] (ascending, -1 padded).
 *   indices[b] is the exact top_k over all positions in both cases.
 * REINDEX: scores only the positions of pool_in[b] (block ids from an
 *   earlier FULL call over the same keys) with this layer's q_idx and
 *   writes the top_k of them to indices[b], in the order pool_in[b] lists
 *   the blocks (increasing when pool_in comes from FULL).  Ids that are
 *   negative or past the sequence are skipped; a repeated id is scored
 *   twice, so its positions may repeat.
 * keys: the layer whose idx_keys are scored; q_idx, w_idx: the query as
 * for csa2_index_scores (scores as defined there); indices: device int32
 * [batch][top_k].
 * top_k in [1, 4096]; pool_block_tokens must be 8 and pool_blocks in
 * [1, 2048]; max_seq_len at most 8,388,608.  Results are deterministic. */
csa2_status csa2_index_select_workspace_size(int32_t batch, int32_t max_seq_len, int32_t top_k,
                                             int32_t pool_blocks, int32_t pool_block_tokens,
                                             size_t *bytes);
csa2_status csa2_index_select(const csa2_kv_layer *keys, const csa2_seqs *seqs, const void *q_idx,
                              const float *w_idx, int32_t top_k, int32_t mode, const int32_t *pool_in, int32_t *pool_out,
                              int32_t pool_blocks, int32_t pool_block_tokens, int32_t *indices,
                              void *ws, size_t ws_bytes, csa2_stream stream);

/* ---- Full-mode selection with this step's appends in the same launch
 * ([P1] "CSA2" Full mode and "Hierarchical Sparse Indexer"; the appended row
 * is the [P1] "FP4 KV cache" entry of the token being decoded, which is
 * visible to this step's selection).  seqs->seq_lens count the new token:
 * for every sequence b with n = seq_lens[b] >= 1, each of the n_appends rows
 * is written at position n - 1 of its layer exactly as csa2_kv_append writes
 * it at position seq_lens[b] (csa2_kv_append with lengths n - 1), and then
 * indices (and pool_out, when not NULL) are what csa2_index_select in FULL
 * mode returns over positions 0 .. n - 1.  When an append writes the scanned
 * layer's keys (the same idx_keys storage, with idx_key given), the new key is
 * scored from that input directly; otherwise the key at n - 1 is read from the
 * cache.  The append workgroups ride in the scan's launch, so no launch is
 * added.  Appends write disjoint storage (no two share codes, or key storage,
 * that both write); 0 <= n_appends <= 8.  Other arguments, limits and the
 * workspace (csa2_index_select_workspace_size) as for csa2_index_select. */
typedef struct {
  const csa2_kv_layer *layer;
  const float *latent;      /* device fp32 [batch][512] or NULL */
  const uint16_t *rope;     /* device bf16 [batch][rope_dim] or NULL */
  const void *idx_key;      /* device [batch][idx_dim] (fp32 for CSA2_FP4 keys, packed here) or NULL */
} csa2_append;
csa2_status csa2_index_select_append(const csa2_kv_layer *keys, const csa2_seqs *seqs, const csa2_append *appends,
                                     int32_t n_appends, const void *q_idx, const float *w_idx, int32_t top_k,
                                     int32_t *pool_out, int32_t pool_blocks, int32_t pool_block_tokens,
                                     int32_t *indices, void *ws, size_t ws_bytes, csa2_stream stream);

/* ---- Reindex for several layers at once ([P1] "CSA2" Reindex mode and
 * "Hierarchical Sparse Indexer": every later selecting layer rescores only
 * the candidate pool of the first Full layer with its own query).  Each entry
 * of `queries` is one REINDEX call of csa2_index_select over the same keys,
 * seqs, pool_in, pool_blocks and top_k: its q_idx / w_idx as defined there and
 * its own indices (device int32 [batch][top_k]).  Results equal those of one
 * csa2_index_select call per layer; the layers' pool scoring runs in one
 * launch and their selections in one more.  1 <= n_layers <= 8.  Workspace
 * from csa2_index_reindex_layers_workspace_size (it holds no per-position
 * keys, so it does not grow with the sequence length). */
typedef struct {
  const void *q_idx;
  const float *w_idx;
  int32_t *indices;
} csa2_reindex_query;
csa2_status csa2_index_reindex_layers_workspace_size(int32_t n_layers, int32_t batch, int32_t top_k,
                                                    int32_t pool_blocks, int32_t pool_block_tokens, size_t *bytes);
csa2_status csa2_index_reindex_layers(const csa2_kv_layer *keys, const csa2_seqs *seqs,
                                      const csa2_reindex_query *queries, int32_t n_layers, int32_t top_k,
                                      const int32_t *pool_in, int32_t pool_blocks, int32_t pool_block_tokens,
                                      void *ws, size_t ws_bytes, csa2_stream stream);

/* ---- Sparse FP4 decode attention ([P1] "CSA2": all heads share one latent;
 * "FP4 KV cache": entries are dequantized before attention; [P4] section 2:
 * 64 heads, 1 KV head).  For each sequence b and head h, over the valid
 * selected positions S = {indices[b][i] : 0 <= indices[b][i] < seq_lens[b]}:
 *   logit_s = softmax_scale * (q[b,h,0:512] . c_s + q[b,h,512:512+rope] . rope_s)
 *   out[b][h] = sum_s softmax(logit)_s * c_s ,  lse[b][h] = log sum_s exp(logit_s)
 * where c_s is the dequantized latent (K = V).  An empty S gives out = 0 and
 * lse = -inf.  q: device bf16 [batch][heads][latent_dim + rope_dim];
 * indices: device int32 [batch][top_k]; out: device fp32 [batch][heads][512];
 * lse: device fp32 [batch][heads] or NULL.  heads must be a positive multiple
 * of 16 (at most 128); top_k in [1, 4096].  The logits and the softmax run in
 * fp32; q and rope enter the matrix cores as fp16, which holds every bf16
 * value of magnitude 2^-14 .. 65504 (and zero) exactly: inside that range the
 * conversion loses nothing.  Smaller magnitudes become fp16 subnormals (an
 * absolute error below 2^-25 per element); larger ones become infinite and
 * make that head's results NaN, so q and rope must stay below 65504 in
 * magnitude (with debug checks on, such values set a device error flag). */
csa2_status csa2_attn_workspace_size(int32_t batch, int32_t heads, int32_t top_k, int32_t latent_dim,
                                     size_t *bytes);
csa2_status csa2_sparse_fp4_decode_attn(const csa2_kv_layer *layer, const csa2_seqs *seqs,
                                        const uint16_t *q, int32_t heads, const int32_t *indices,
                                        int32_t top_k, float softmax_scale, float *out, float *lse,
                                        void *ws, size_t ws_bytes, csa2_stream stream);

/* ---- The same attention with the sliding-window branch in one softmax
 * ([P1] "KV bottleneck" and "Causal Encoder-Decoder": a local window of 128
 * beside the global branch; "FP4 KV cache": the window stays FP8).  The
 * result equals csa2_sparse_fp4_decode_attn followed by csa2_swa_attn_merge
 * with seq_lens = seqs->seq_lens (up to rounding): out and lse are the
 * attention over the union of the selected entries and the window slots
 * holding positions max(0, n - 128) .. n - 1, n = seqs->seq_lens[b]; the
 * window contributes logits to the latent part of q only.  The window's 128
 * slots run as four more split workgroups of the same kernel, so no second
 * attention pass and no in-place merge are needed.  win: the ring (win->batch
 * >= seqs->batch).  new_latent: NULL, or device fp32 [batch][512], the
 * current token's window entry: it is packed into slot (n - 1) mod 128 of
 * the ring first (as csa2_swa_append with positions n - 1 would; sequences
 * with n <= 0 take none) and attended in the same call.  Other arguments and
 * limits as for csa2_sparse_fp4_decode_attn; workspace from
 * csa2_attn_swa_workspace_size. */
csa2_status csa2_attn_swa_workspace_size(int32_t batch, int32_t heads, int32_t top_k, int32_t latent_dim,
                                         size_t *bytes);
csa2_status csa2_sparse_fp4_decode_attn_swa(const csa2_kv_layer *layer, const csa2_seqs *seqs,
                                            const uint16_t *q, int32_t heads, const int32_t *indices,
                                            int32_t top_k, float softmax_scale, const csa2_swa_window *win,
                                            const float *new_latent, float *out, float *lse, void *ws,
                                            size_t ws_bytes, csa2_stream stream);

/* ---- The attention of several layers in one launch ([P1] "CSA2": the
 * decoder's layers each attend over their own KV with indices that a Full or
 * Reindex layer selected, a Reuse layer taking another layer's indices
 * unchanged; [P1] "Hierarchical Sparse Indexer": a step runs one Full and
 * several Reindex layers).  Every entry of `layers` is one problem exactly as
 * csa2_sparse_fp4_decode_attn defines it -- its own KV pool, query (device
 * bf16 [batch][heads][512 + rope_dim]), indices (device int32
 * [batch][top_k]), out (device fp32 [batch][heads][512]) and lse (device fp32
 * [batch][heads] or NULL) -- or, with `win` set, as
 * csa2_sparse_fp4_decode_attn_swa defines it (its own ring; new_latent NULL
 * or that layer's current window entry).  All layers share seqs, heads,
 * top_k and softmax_scale; their pools have the same rope_dim; either every
 * layer has a window or none has.  1 <= n_layers <= 20, and n_layers *
 * seqs->batch at most 65,535 (the launch's (layer, sequence) grid dimension;
 * larger calls fail with CSA2_ERR_INVALID_ARG).  Results equal those
 * of one call per layer (the same kernels; only the launch is shared), so the
 * layers' problems are independent: no output may alias another layer's
 * input.  Workspace from csa2_attn_layers_workspace_size (with_window: 1 when
 * the layers have windows). */
typedef struct {
  const csa2_kv_layer *layer;
  const uint16_t *q;
  const int32_t *indices;
  float *out;
  float *lse;
  const csa2_swa_window *win; /* NULL: no sliding-window branch */
  const float *new_latent;    /* with win: NULL or device fp32 [batch][512] */
} csa2_attn_layer;
csa2_status csa2_attn_layers_workspace_size(int32_t n_layers, int32_t batch, int32_t heads, int32_t top_k,
                                            int32_t latent_dim, int32_t with_window, size_t *bytes);
csa2_status csa2_sparse_fp4_decode_attn_layers(const csa2_attn_layer *layers, int32_t n_layers,
                                               const csa2_seqs *seqs, int32_t heads, int32_t top_k,
                                               float softmax_scale, void *ws, size_t ws_bytes, csa2_stream stream);

/* ---- For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * csa2_sparse_fp4_decode_attn_layers without a workspace argument.  The split
 * partials go to a scratch array the library holds on every device it runs on
 * (32 MiB each, held until the process ends).  When the partials of the usual
 * split count (the size csa2_attn_layers_workspace_size reports) need more,
 * the entries are split over fewer workgroups until they fit; a problem that
 * does not fit even so returns CSA2_ERR_WORKSPACE and launches nothing.  Every
 * call on one device shares
 * that device's scratch: calls that overlap in time on one device (on
 * different streams) race, so serialize them.  The scratch needs no clearing
 * (every partial is written before it is read).  The first call on a device
 * resolves the scratch's address there (not a stream operation; make that
 * first call outside graph capture).  Results equal those of
 * csa2_sparse_fp4_decode_attn_layers on the same arguments (within the
 * rounding of a different split where fewer splits were needed).  Nothing is
 * allocated by this call. */
csa2_status csa2_sparse_fp4_decode_attn_layers_noalloc(const csa2_attn_layer *layers, int32_t n_layers,
                                                       const csa2_seqs *seqs, int32_t heads, int32_t top_k,
                                                       float softmax_scale, csa2_stream stream);

/* ---- Host-side page allocator (no device memory): a free list of block ids
 * [0, num_blocks).  Not thread-safe; one instance per owner. */
typedef struct csa2_block_pool csa2_block_pool;
csa2_block_pool *csa2_block_pool_create(int32_t num_blocks);
/* Takes n ids (n >= 0) into ids_out; fails without taking any when fewer are free. */
csa2_status csa2_block_alloc(csa2_block_pool *pool, int32_t n, int32_t *ids_out);
/* Returns n ids; fails without returning any on an out-of-range or already free id. */
csa2_status csa2_block_free(csa2_block_pool *pool, int32_t n, const int32_t *ids);
int32_t csa2_block_pool_num_free(const csa2_block_pool *pool);
void csa2_block_pool_destroy(csa2_block_pool *pool);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
