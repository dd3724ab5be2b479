// The decode-time append of one token's row to a paged KV pool, shared by the
// standalone append kernel and the append workgroups of the Full-mode scan.
//
// Format: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "FP4 KV
// cache" (E2M1 elements, one E4M3 scale per 16 channels).  The paged layout
// (64-token pages through a block table) is this library's.
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa2 {

// Threads t = 0 .. 63 of the caller write sequence b's row at position
// seq_lens[b] + p_offset: threads 0..31 pack the 32 groups of the 512-channel
// latent; threads 32..63 copy the rope side-band and the indexer key
// (threads 32..39 pack an FP4 key).  Every operand is read before the slot is
// known (none depends on it), so the operand loads are in flight together
// with the two table reads.  A position whose page is not mapped is skipped.
__device__ __forceinline__ void append_row(const KvLayerDev &L, const SeqsDev &S, int b, int p_offset,
                                           const float *__restrict__ latent, const uint16_t *__restrict__ rope,
                                           const void *__restrict__ idx_key, int t, uint32_t *dbg) {
  constexpr int kKey4 = 128;  // FP4 indexer key dims
  const int u = t - kLatent / kGroup;  // 0..31 in the upper half
  const bool has_key = idx_key != nullptr && L.idx_keys != nullptr;
  const float *gsrc = nullptr;  // the 16 values this thread packs, if any
  if (u < 0) {
    if (latent != nullptr) gsrc = latent + (int64_t)b * kLatent + t * kGroup;
  } else if (has_key && L.idx_fp4 && u < kKey4 / kGroup) {
    gsrc = static_cast<const float *>(idx_key) + (int64_t)b * kKey4 + u * kGroup;
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = gsrc != nullptr ? gsrc[i] : 0.f;
  if (dbg != nullptr) {
    bool fin = true;
#pragma unroll
    for (int i = 0; i < 16; ++i) fin &= isfinite(v[i]);
    if (!fin) dbg_raise(dbg, kDbgNonFinite);
  }
  const bool copy_rope = u >= 0 && rope != nullptr && L.rope_dim != 0;  // rope_dim is 64
  uint16_t r0 = 0, r1 = 0;
  if (copy_rope) {
    r0 = rope[(int64_t)b * 64 + u];
    r1 = rope[(int64_t)b * 64 + u + 32];
  }
  const bool copy_key = u >= 0 && has_key && !L.idx_fp4;  // dims u and u + 32 of 64
  uint32_t k0 = 0, k1 = 0;
  if (copy_key) {
    if (L.idx_f32) {
      const uint32_t *src = static_cast<const uint32_t *>(idx_key) + (int64_t)b * kIdxDim;
      k0 = src[u];
      k1 = src[u + 32];
    } else {
      const uint16_t *src = static_cast<const uint16_t *>(idx_key) + (int64_t)b * kIdxDim;
      k0 = src[u];
      k1 = src[u + 32];
    }
  }

  const int p = S.seq_lens[b] + p_offset;
  if (p < 0) return;
  const int page = p / kPage;
  if (page >= S.max_blocks) return;
  const int blk = S.block_table[(int64_t)b * S.max_blocks + page];
  if (blk < 0 || blk >= L.num_blocks) return;
  const int64_t slot = (int64_t)blk * kPage + p % kPage;
  if (gsrc != nullptr) {
    uint32_t w0, w1;
    const uint32_t sc = pack_group16(v, &w0, &w1);
    if (u < 0) {
      reinterpret_cast<uint2 *>(L.codes + slot * (kLatent / 2))[t] = make_uint2(w0, w1);
      L.scales[slot * (kLatent / kGroup) + t] = (uint8_t)sc;
    } else {
      reinterpret_cast<uint2 *>(static_cast<uint8_t *>(L.idx_keys) + slot * (kKey4 / 2))[u] = make_uint2(w0, w1);
      L.idx_scales[slot * (kKey4 / kGroup) + u] = (uint8_t)sc;
    }
  }
  if (copy_rope) {
    L.rope[slot * 64 + u] = r0;
    L.rope[slot * 64 + u + 32] = r1;
  }
  if (copy_key) {
    if (L.idx_f32) {
      uint32_t *dst = static_cast<uint32_t *>(L.idx_keys) + slot * kIdxDim;
      dst[u] = k0;
      dst[u + 32] = k1;
    } else {
      uint16_t *dst = static_cast<uint16_t *>(L.idx_keys) + slot * kIdxDim;
      dst[u] = (uint16_t)k0;
      dst[u + 32] = (uint16_t)k1;
    }
  }
}

}  // namespace csa2
