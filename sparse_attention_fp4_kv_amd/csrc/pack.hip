// FP4 pack / unpack / paged append kernels.
//
// Format: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "FP4 KV
// cache" (E2M1 elements, one E4M3 scale per 16 channels).  The pack is
// HBM-bound (reads 4 B per channel, writes 0.5625 B per channel): one thread
// owns one 16-channel group, so a wave reads 64 contiguous 64-byte runs and
// writes 64 contiguous 8-byte runs plus 64 scale bytes.
#include "common.h"
#include "kernels.h"

namespace csa2 {

__global__ void __launch_bounds__(256) fp4_pack_kernel(const float *__restrict__ x, int64_t n_groups,
                                                       uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const float4 *src = reinterpret_cast<const float4 *>(x + g * kGroup);
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = src[i];
    v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  uint32_t w0, w1;
  const uint32_t sc = pack_group16(v, &w0, &w1);
  reinterpret_cast<uint2 *>(codes)[g] = make_uint2(w0, w1);
  scales[g] = (uint8_t)sc;
}

__global__ void __launch_bounds__(256) fp4_unpack_kernel(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         int64_t n_groups, float *__restrict__ y) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const uint2 w = reinterpret_cast<const uint2 *>(codes)[g];
  const float s = e4m3_decode(scales[g]);
  float4 *dst = reinterpret_cast<float4 *>(y + g * kGroup);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = i < 2 ? w.x : w.y;
    const int sh = 16 * (i & 1);
    float4 f;
    f.x = e2m1_decode(word >> sh) * s;
    f.y = e2m1_decode(word >> (sh + 4)) * s;
    f.z = e2m1_decode(word >> (sh + 8)) * s;
    f.w = e2m1_decode(word >> (sh + 12)) * s;
    dst[i] = f;
  }
}

// One workgroup of 64 threads per sequence: threads 0..31 pack the 32 groups
// of the 512-channel latent into the slot of position seq_lens[b]; the rest
// copy the rope side-band and the indexer key (threads 32..39 pack an FP4 key).
// Every operand is read before the slot is known (none depends on it), so the
// operand loads are in flight together with the two table reads.
__global__ void __launch_bounds__(64) kv_append_kernel(KvLayerDev L, SeqsDev S, const float *__restrict__ latent,
                                                       const uint16_t *__restrict__ rope,
                                                       const void *__restrict__ idx_key) {
  constexpr int kKey4 = 128;  // FP4 indexer key dims
  const int b = blockIdx.x;
  const int t = threadIdx.x;
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

  const int p = S.seq_lens[b];
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

__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t *__restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fp4_pack(const float *x, int64_t rows, int channels, uint8_t *codes, uint8_t *scales,
                           hipStream_t st) {
  const int64_t n = rows * (channels / kGroup);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  timer_before(kKernFp4Pack, st);
  fp4_pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, n, codes, scales);
  timer_after(kKernFp4Pack, st);
  return hipGetLastError();
}

hipError_t launch_fp4_unpack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int channels, float *y,
                             hipStream_t st) {
  const int64_t n = rows * (channels / kGroup);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fp4_unpack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(codes, scales, n, y);
  return hipGetLastError();
}

hipError_t launch_kv_append(const KvLayerDev &L, const SeqsDev &S, const float *latent, const uint16_t *rope,
                            const void *idx_key, hipStream_t st) {
  if (S.batch == 0) return hipSuccess;
  timer_before(kKernKvAppend, st);
  kv_append_kernel<<<dim3(S.batch), dim3(64), 0, st>>>(L, S, latent, rope, idx_key);
  timer_after(kKernKvAppend, st);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<uint32_t *>(p), words);
  return hipGetLastError();
}

}  // namespace csa2
