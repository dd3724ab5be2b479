// Finishing KV latents before they are cached (RMSNorm, RoPE, FP4 pack) and
// the FP4 indexer key projected from the cached entry.
//
// Sources: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "FP4 KV
// cache" (the 512-channel latent is RMS-normalised and rotated by RoPE, which
// keeps its norm, before it is stored as E2M1 + one E4M3 scale per 16
// channels), and section "CSA2" (a Full layer's indexer K is a projection of
// the main KV; 32 indexer heads of dimension 128; V4 keeps indexer keys in
// FP4).
//
// This library's reading of the open points:
//   y = x / sqrt(mean(x^2) + eps) * gamma over the 512 channels;
//   RoPE turns channels 448 + 2i, 449 + 2i (i < 32) by fl32(p * f_i),
//   f_i = fl32(theta^(-2i/64));
//   k = W_idx x_hat, x_hat the dequantized FP4 entry, W_idx bf16 [128][512],
//   k stored in the same FP4 format (128 dims: 64 code bytes + 8 scales).
//
// Design: a workgroup (4 waves) finishes 32 rows.  A wave takes one row at a
// time, lane l holding channels 8l .. 8l+7: the sum of squares is a wave
// reduction, lanes 56..63 hold the 64 rotated channels, and each 16-channel
// group is two neighbouring lanes (amax by one lane swap), so the codes of a
// row leave as one 4-byte store per lane.  The dequantized entry (exact in
// bf16: at most 6 significant bits) is parked in LDS; the projection is one
// v_mfma_f32_32x32x16_bf16 chain per wave (M = the 32 rows, N = 32 of the
// 128 key dims, 32 k-steps), and the keys are packed from LDS, one 16-dim
// group per thread.
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int kRows = 32;                     // rows per workgroup
constexpr int kRopeFirst = kLatent - 64;      // 448
constexpr int kKeyDim = 128;                  // indexer key dims
constexpr int kLdX = kLatent + 8;             // bf16 per LDS row of the dequantized entries
constexpr int kLdK = kKeyDim + 4;             // fp32 per LDS row of the keys

// Where row r of a launch comes from and goes to.
struct RowMap {
  // rows mode (CED / standalone): row r = layer * tokens + t, inputs and outputs contiguous
  int64_t tokens;
  int64_t pos0;
  // paged mode (append): row = sequence b, destination slot from the page table
  int paged;
  KvLayerDev L;
  SeqsDev S;
};

struct FinishArgs {
  const float *c;        // raw latents [rows][512]
  int64_t rows;
  const float *gamma;    // [layers][512]
  float eps;
  float theta;           // 0: no rotation
  const uint16_t *w_idx; // [layers][128][512] bf16 or null
  uint8_t *codes;        // rows mode: [rows][256]
  uint8_t *scales;       // rows mode: [rows][32]
  uint8_t *k_codes;      // rows mode: [rows][64]
  uint8_t *k_scales;     // rows mode: [rows][8]
  float *x_f32;          // rows mode, optional: [rows][512] finished latent before packing
  float *k_f32;          // rows mode, optional: [rows][128] key before packing
  RowMap m;
};

// Destination slot of row r (-1: not stored), its token position and layer.
__device__ __forceinline__ int64_t row_slot(const FinishArgs &a, int64_t r, int64_t *pos, int *layer) {
  if (!a.m.paged) {
    *layer = (int)(r / a.m.tokens);
    *pos = a.m.pos0 + r % a.m.tokens;
    return r;
  }
  *layer = 0;
  const int p = a.m.S.seq_lens[r];
  *pos = p < 0 ? 0 : p;
  if (p < 0) return -1;
  const int page = p / kPage;
  if (page >= a.m.S.max_blocks) return -1;
  const int blk = a.m.S.block_table[r * a.m.S.max_blocks + page];
  if (blk < 0 || blk >= a.m.L.num_blocks) return -1;
  return (int64_t)blk * kPage + p % kPage;
}

// Sum over the wave through DPP row shifts and broadcasts (VALU only; a
// __shfl_xor butterfly costs one LDS round trip per step).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0x111>(v);
  v += dpp_f32<0x112>(v);
  v += dpp_f32<0x114>(v);
  v += dpp_f32<0x118>(v);
  v += __uint_as_float(dpp_u32<0x142, 0xA>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x143, 0xC>(__float_as_uint(v)));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

__device__ __forceinline__ uint16_t exact_bf16(float v) { return (uint16_t)(__float_as_uint(v) >> 16); }

// EARLY: every W_idx fragment of the key projection is loaded at the start,
// in flight together with the rows (the decode-time append of a few rows,
// where those loads are the critical path); otherwise they stream 8 k-steps
// ahead of the MFMA chain, which keeps registers for occupancy in bulk runs.
template <bool EARLY>
__global__ void __launch_bounds__(256) finish_kernel(FinishArgs a) {
  // the dequantized rows, then (after every wave's projection has read them)
  // the projected keys: one LDS area, so four workgroups fit a CU
  __shared__ __attribute__((aligned(16))) union {
    uint16_t xs[kRows][kLdX];
    float ks[kRows][kLdK];
  } sx;
  auto &xs = sx.xs;
  auto &ks = sx.ks;
  __shared__ int64_t slots[kRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = a.m.paged ? (int64_t)blockIdx.x * kRows
                                 : (int64_t)blockIdx.y * a.m.tokens + (int64_t)blockIdx.x * kRows;
  const int64_t row_end = a.m.paged ? a.rows : (int64_t)(blockIdx.y + 1) * a.m.tokens;
  const int layer = a.m.paged ? 0 : (int)blockIdx.y;
  constexpr int kSteps = kLatent / 16;  // 32 k-steps of the key projection
  constexpr int kAhead = EARLY ? kSteps : 8;
  // k[r][n] = sum_c x_hat[r][c] W[n][c]: wave w owns n in [32w, 32w + 32)
  const uint16_t *wrow = a.w_idx == nullptr ? nullptr
                         : a.w_idx + ((size_t)layer * kKeyDim + 32 * wave + (lane & 31)) * kLatent + 8 * (lane >> 5);
  uint4 wb[kAhead];
  if (EARLY && wrow != nullptr) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) wb[i] = *reinterpret_cast<const uint4 *>(wrow + 16 * i);
  }
  const float *gam = a.gamma + (size_t)layer * kLatent + 8 * lane;
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = gam[i];
  // RoPE cos / sin of the wave's 8 rows spread over all its lanes: lane 8 j + m
  // computes pairs 4 m .. 4 m + 3 of row j (angle fl32(p * fl32(theta^(-2i/64)))),
  // and the rotating lanes 56 + m fetch them when row j is finished
  const bool rope = a.theta != 0.0f;
  const bool rot = rope && lane >= kRopeFirst / 8;
  float rc[4] = {1.0f, 1.0f, 1.0f, 1.0f}, rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (rope && row0 + wave < row_end) {  // (uniform: a wave whose rows are all past the end skips it)
    const int64_t r = row0 + 4 * (lane >> 3) + wave;
    int64_t p = 0;
    if (r < row_end) {
      if (a.m.paged) {
        const int sp = a.m.S.seq_lens[r];
        p = sp < 0 ? 0 : sp;
      } else {
        p = a.m.pos0 + r % a.m.tokens;
      }
    }
    const float pf = (float)p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * (lane & 7) + q;
      const float fq = (float)pow((double)a.theta, -2.0 * i / 64.0);
      const float t = pf * fq;
      if constexpr (EARLY) {
        // few rows: the fp32 angle reduced by 2 pi in double (2 pi as a double
        // plus its remainder; |k| < 2^23) and the small-argument double
        // sincos, so no large-argument reduction table is read from memory
        constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
        const double td = (double)t;
        const double k = rint(td * (1.0 / kTwoPiHi));
        const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, td));
        double sd, cd;
        sincos(r, &sd, &cd);
        rs[q] = (float)sd;
        rc[q] = (float)cd;
      } else {
        sincosf(t, &rs[q], &rc[q]);
      }
    }
  }
  // a wave's rows are 4 apart; the next one's channels are loaded while this
  // one is finished
  auto load_row = [&](int64_t r, float (&x)[8]) {
    const float4 *src = reinterpret_cast<const float4 *>(a.c + r * kLatent + 8 * lane);
    const float4 u = src[0], v = src[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  };
  float xn[8];
  if (row0 + wave < row_end) load_row(row0 + wave, xn);
  for (int j = 0; j < kRows / 4; ++j) {
    const int lr = 4 * j + wave;  // local row
    const int64_t r = row0 + lr;
    if (r >= row_end) {  // uniform over the wave (and so are the later rows); their keys come from stale LDS and are never stored
      if (lane == 0) slots[lr] = -1;
      continue;
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = xn[i];
    if (j + 1 < kRows / 4 && r + 4 < row_end) load_row(r + 4, xn);
    int64_t pos = 0;
    int lay = 0;
    const int64_t slot = row_slot(a, r, &pos, &lay);
    if (lane == 0) slots[lr] = slot;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
    ss = wave_sum(ss);
    const float inv = __fdiv_rn(1.0f, __fsqrt_rn(ss * (1.0f / kLatent) + a.eps));
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (x[i] * inv) * g[i];
    if (rope) {  // uniform: every lane takes part in the fetch
      const int src = 8 * j + (lane & 7);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float c = __shfl(rc[q], src), s = __shfl(rs[q], src);
        if (rot) {
          const float u = x[2 * q], v = x[2 * q + 1];
          x[2 * q] = u * c - v * s;
          x[2 * q + 1] = u * s + v * c;
        }
      }
    }
    // pack: group 16 channels = lanes 2m, 2m+1
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, dpp_f32<0xB1>(amax));  // the group's other lane (quad_perm 1,0,3,2)
    const uint32_t sc = e4m3_encode(__fdiv_rn(amax, 6.0f));
    const float s = e4m3_decode(sc);
    uint32_t word = 0u;
    uint16_t xb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t nib = sc ? (((__float_as_uint(x[i]) >> 31) << 3) | e2m1_magnitude(fabsf(x[i]), s)) : 0u;
      word |= nib << (4 * i);
      xb[i] = exact_bf16(e2m1_decode(nib) * s);
    }
    uint4 xv;
    xv.x = xb[0] | ((uint32_t)xb[1] << 16);
    xv.y = xb[2] | ((uint32_t)xb[3] << 16);
    xv.z = xb[4] | ((uint32_t)xb[5] << 16);
    xv.w = xb[6] | ((uint32_t)xb[7] << 16);
    *reinterpret_cast<uint4 *>(&xs[lr][8 * lane]) = xv;
    if (slot >= 0) {
      uint8_t *codes = a.m.paged ? a.m.L.codes : a.codes;
      uint8_t *scales = a.m.paged ? a.m.L.scales : a.scales;
      reinterpret_cast<uint32_t *>(codes + slot * (kLatent / 2))[lane] = word;
      if ((lane & 1) == 0) scales[slot * (kLatent / kGroup) + (lane >> 1)] = (uint8_t)sc;
      if (a.x_f32 != nullptr) {
        float4 *dst = reinterpret_cast<float4 *>(a.x_f32 + slot * kLatent + 8 * lane);
        dst[0] = make_float4(x[0], x[1], x[2], x[3]);
        dst[1] = make_float4(x[4], x[5], x[6], x[7]);
      }
    }
  }
  if (a.w_idx == nullptr) return;  // uniform over the workgroup
  __syncthreads();
  {
    const uint16_t *xrow = &xs[lane & 31][8 * (lane >> 5)];
    f32x16 acc = {};
    if (!EARLY) {
#pragma unroll
      for (int i = 0; i < kAhead; ++i) wb[i] = *reinterpret_cast<const uint4 *>(wrow + 16 * i);
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const uint4 wv = wb[ks % kAhead];
      if (ks + kAhead < kSteps) wb[ks % kAhead] = *reinterpret_cast<const uint4 *>(wrow + 16 * (ks + kAhead));
      const uint4 xv = *reinterpret_cast<const uint4 *>(xrow + 16 * ks);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv), __builtin_bit_cast(bf16x8, wv),
                                                    acc, 0, 0, 0);
    }
    __syncthreads();  // every wave has read xs (the keys take its place)
#pragma unroll
    for (int e = 0; e < 16; ++e) ks[8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][32 * wave + (lane & 31)] = acc[e];
  }
  __syncthreads();
  {
    const int lr = tid >> 3, g8 = tid & 7;  // 32 rows x 8 groups
    const int64_t slot = slots[lr];
    if (slot < 0) return;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = ks[lr][16 * g8 + i];
    uint32_t w0, w1;
    const uint32_t sc = pack_group16(v, &w0, &w1);
    uint8_t *kc = a.m.paged ? static_cast<uint8_t *>(a.m.L.idx_keys) : a.k_codes;
    uint8_t *kscl = a.m.paged ? a.m.L.idx_scales : a.k_scales;
    reinterpret_cast<uint2 *>(kc + slot * (kKeyDim / 2))[g8] = make_uint2(w0, w1);
    kscl[slot * (kKeyDim / kGroup) + g8] = (uint8_t)sc;
    if (a.k_f32 != nullptr) {
      float4 *dst = reinterpret_cast<float4 *>(a.k_f32 + slot * kKeyDim + 16 * g8);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  }
}

}  // namespace

hipError_t launch_kv_finish_rows(const float *c, int64_t tokens, int n_layers, int64_t pos0, const KvFinish &fin,
                                 uint8_t *codes, uint8_t *scales, uint8_t *k_codes, uint8_t *k_scales, float *x_f32,
                                 float *k_f32, hipStream_t st) {
  if (tokens == 0 || n_layers == 0) return hipSuccess;
  FinishArgs a{};
  a.c = c;
  a.rows = tokens * n_layers;
  a.gamma = fin.gamma;
  a.eps = fin.eps;
  a.theta = fin.theta;
  a.w_idx = fin.w_idx;
  a.codes = codes;
  a.scales = scales;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.x_f32 = x_f32;
  a.k_f32 = k_f32;
  a.m.tokens = tokens;
  a.m.pos0 = pos0;
  a.m.paged = 0;
  const dim3 grid((unsigned)((tokens + kRows - 1) / kRows), (unsigned)n_layers);
  timer_before(kKernKvFinish, st);
  finish_kernel<false><<<grid, dim3(256), 0, st>>>(a);
  timer_after(kKernKvFinish, st);
  return hipGetLastError();
}

hipError_t launch_kv_append_finish(const KvLayerDev &L, const SeqsDev &S, const float *latent, const KvFinish &fin,
                                   hipStream_t st) {
  if (S.batch == 0) return hipSuccess;
  FinishArgs a{};
  a.c = latent;
  a.rows = S.batch;
  a.gamma = fin.gamma;
  a.eps = fin.eps;
  a.theta = fin.theta;
  a.w_idx = fin.w_idx;
  a.m.paged = 1;
  a.m.L = L;
  a.m.S = S;
  const dim3 grid((unsigned)((S.batch + kRows - 1) / kRows));
  timer_before(kKernKvAppend, st);
  finish_kernel<true><<<grid, dim3(256), 0, st>>>(a);
  timer_after(kKernKvAppend, st);
  return hipGetLastError();
}

}  // namespace csa2
