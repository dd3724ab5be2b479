// The sliding-window (SWA) branch: FP8 window entries and their attention,
// merged into the global branch's result.
//
// Sources: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, sections "KV
// bottleneck" (a local sliding-window branch beside the global one),
// "Causal Encoder-Decoder" (window n_win = 128) and "FP4 KV cache" (the
// quantization-sensitive SWA KV stays in FP8).
//
// This library's reading of the open points: a window entry is the layer's
// 512-channel local latent (key = value, no rope part); FP8 is E4M3FN with
// one fp32 scale per token, s = amax / 448, code = E4M3_RNE(x / s); the
// window of n positions is positions n-128 .. n-1 in a ring of 128 slots
// (slot = position mod 128); the branches are one softmax over the union of
// their entries, i.e. the lse-weighted merge of the two results.
//
// Design: the attention of one sequence's window is small (128 entries x up
// to 128 heads), so one workgroup serves 16 heads of one sequence and holds
// the whole window: QK^T is v_mfma_f32_16x16x32_f16 with the FP8 codes
// converted to fp16 in registers (exact; the per-token scale is applied to
// the logit), an exact softmax over the 128 logits, and PV with P times the
// token's scale (normalized by a power of two so it stays in fp16's normal
// range) as fp16 hi + lo parts against the window staged in LDS as fp16, 256
// channels at a time, read through transposing LDS loads.  The epilogue
// merges with the global result (out, lse) in place.  This pair of kernels
// serves a caller that already holds the global result; the decode path runs
// the window inside the global attention launch instead (attention.hip: the
// ring's tiles as extra split workgroups, the append done there too).
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int kWin = 128;          // window slots
constexpr int kHg = 16;            // heads per workgroup
constexpr int kQLd = kLatent + 8;  // f16 per LDS query row
constexpr int kVLd = 256 + 8;      // f16 per LDS window row (one half of the channels)
constexpr int kPLd = kWin + 8;

struct SwaArgs {
  const uint8_t *codes;  // [B][128][512]
  const float *scales;   // [B][128]
  const int32_t *lens;   // [B] positions of each sequence, current token included
  const uint16_t *q;     // [B][H][qdim] bf16
  int heads, qdim;
  float scale_log2;      // softmax scale * log2(e)
  float *out;            // [B][H][512], in/out
  float *lse;            // [B][H], in/out
};

struct __attribute__((aligned(16))) SwaSmem {
  __attribute__((aligned(16))) f16 q[kHg][kQLd];
  __attribute__((aligned(16))) f16 v[kWin][kVLd];
  float s[kHg][kWin + 1];
  __attribute__((aligned(16))) f16 p_hi[kHg][kPLd];
  __attribute__((aligned(16))) f16 p_lo[kHg][kPLd];
  float tok_scale[kWin];
  float lse_g[kHg], lse_s[kHg], inv_l[kHg];
  float unnorm;  // the power of two that P was multiplied by, inverted
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// PV operand (B of v_mfma_f32_16x16x32_f16: k = entries, n = channels) from
// the row-major window with two transposing loads: within 16 lanes,
// ds_read_b64_tr_b16 gives lane i element i % 4 of the 8-byte chunks read by
// lanes 4 e + i / 4, so lane L of k-group g = L / 16 points at row
// 8 g + (L / 4) % 4 (+ 4 for the second load), channels n0 + 4 (L % 4) .. + 3.
__device__ __forceinline__ f16x8 window_operand(const f16 *p) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * kVLd));
  const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(f16x8, ab);
}

template <int G>
__device__ __forceinline__ float grp_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}
template <int G>
__device__ __forceinline__ float grp_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);
  return v;
}

__global__ void __launch_bounds__(256) swa_attn_kernel(SwaArgs a) {
  __shared__ SwaSmem sm;
  const int b = blockIdx.x, h0 = blockIdx.y * kHg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.lens[b];
  const int nwin = n <= 0 ? 0 : (n < kWin ? n : kWin);  // valid slots: 0 .. nwin-1
  if (nwin == 0) return;  // an empty window leaves the global result as it is
  const uint8_t *win = a.codes + (size_t)b * kWin * kLatent;
  // ---- query tile (bf16 -> fp16), token scales, global lse
  {
    const int h = tid >> 4, c0 = 32 * (tid & 15);
    const uint4 *src = reinterpret_cast<const uint4 *>(a.q + ((size_t)b * a.heads + h0 + h) * a.qdim + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      f16x8 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[2 * j] = (f16)__uint_as_float(w[j] << 16);
        r[2 * j + 1] = (f16)__uint_as_float(w[j] & 0xFFFF0000u);
      }
      *reinterpret_cast<f16x8 *>(&sm.q[h][c0 + 8 * i]) = r;
    }
    if (tid < kWin) sm.tok_scale[tid] = tid < nwin ? a.scales[(size_t)b * kWin + tid] : 0.0f;
    if (tid < kHg) sm.lse_g[tid] = a.lse[(size_t)b * a.heads + h0 + tid];
  }
  // Every global read of the kernel is issued here, so one memory latency
  // covers them all: the B fragments of QK^T (wave w owns entries
  // 32w .. 32w+31), this thread's share of the window for the PV staging
  // (slot tid / 2, channels 128 (tid % 2) .. + 127 of each half) and the
  // global result this lane merges into.
  uint2 kb[2][16];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int e = 32 * wave + 16 * nb + (lane & 15);
    const uint8_t *row = win + (size_t)(e < nwin ? e : 0) * kLatent + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) kb[nb][kk] = *reinterpret_cast<const uint2 *>(row + 32 * kk);
  }
  const int se = tid >> 1, sc0 = 128 * (tid & 1);
  uint4 raw[2][8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint4 *src = reinterpret_cast<const uint4 *>(win + (size_t)(se < nwin ? se : 0) * kLatent + 256 * half + sc0);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[half][i] = src[i];
  }
  float og[2][4][4];  // global out of (half, nb, i): head 4 (lane / 16) + i, channel 256 half + 64 wave + 16 nb + lane % 16
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        og[half][nb][i] = a.out[((size_t)b * a.heads + h0 + 4 * (lane >> 4) + i) * kLatent + 256 * half + 64 * wave +
                                16 * nb + (lane & 15)];
  __syncthreads();
  // ---- logits (log2 domain), masked past the window
  {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const f16x8 qa = *reinterpret_cast<const f16x8 *>(&sm.q[lane & 15][32 * kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, fp8x8_to_f16(kb[nb][kk]), acc[nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int e = 32 * wave + 16 * nb + (lane & 15);
      const float ts = sm.tok_scale[e] * a.scale_log2;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.s[4 * (lane >> 4) + i][e] = e < nwin ? acc[nb][i] * ts : -INFINITY;
    }
  }
  __syncthreads();
  // ---- exact softmax per head (16 lanes per head, 8 entries per lane); P times the token scale
  {
    const int h = tid >> 4, e0 = 8 * (tid & 15);
    float sv[8], ts[8];
    float mx = -INFINITY, smax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = sm.s[h][e0 + i];
      ts[i] = sm.tok_scale[e0 + i];
      mx = fmaxf(mx, sv[i]);
      smax = fmaxf(smax, ts[i]);
    }
    mx = grp_max<16>(mx);
    smax = grp_max<16>(smax);
    // a power of two that brings the largest token scale into [1, 2): P stays in fp16's normal range
    const float norm = smax > 0.0f ? __uint_as_float((254u - ((__float_as_uint(smax) >> 23) & 0xFFu)) << 23) : 1.0f;
    float l = 0.0f;
    f16 ph[8], pl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = e0 + i < nwin ? exp2f(sv[i] - mx) : 0.0f;
      l += p;
      // pv is rounded to fp32 once and both parts are split from that value
      // (left visible, the product gets folded into one fp16 conversion but
      // not the other, and hi + lo can miss pv by one fp16 ulp of hi)
      float pv = p * (ts[i] * norm);
      asm volatile("" : "+v"(pv));
      ph[i] = (f16)pv;
      pl[i] = (f16)(pv - (float)ph[i]);
    }
    l = grp_sum<16>(l);
    f16x8 vh, vl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vh[i] = ph[i];
      vl[i] = pl[i];
    }
    *reinterpret_cast<f16x8 *>(&sm.p_hi[h][e0]) = vh;
    *reinterpret_cast<f16x8 *>(&sm.p_lo[h][e0]) = vl;
    if ((tid & 15) == 0) {
      sm.inv_l[h] = 1.0f / l;
      sm.lse_s[h] = (mx + log2f(l)) * 0.6931471805599453f;
    }
    if (tid == 0) sm.unnorm = 1.0f / norm;
  }
  // ---- PV over two halves of the channels, merged into the global result
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // P and the softmax state written / the previous half's reads of v done
    {
      // stage channels 256 half .. +255 of every slot as fp16 (zeros past the window)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 r = raw[half][i];
        f16x8 lo = fp8x8_to_f16(make_uint2(r.x, r.y));
        f16x8 hi = fp8x8_to_f16(make_uint2(r.z, r.w));
        if (se >= nwin) lo = hi = f16x8{};
        *reinterpret_cast<f16x8 *>(&sm.v[se][sc0 + 16 * i]) = lo;
        *reinterpret_cast<f16x8 *>(&sm.v[se][sc0 + 16 * i + 8]) = hi;
      }
    }
    __syncthreads();
    f32x4 o[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                  f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kWin / 32; ++ks) {
      const f16x8 ah = *reinterpret_cast<const f16x8 *>(&sm.p_hi[lane & 15][32 * ks + 8 * (lane >> 4)]);
      const f16x8 al = *reinterpret_cast<const f16x8 *>(&sm.p_lo[lane & 15][32 * ks + 8 * (lane >> 4)]);
      const f16 *base = &sm.v[32 * ks + 8 * (lane >> 4) + ((lane >> 2) & 3)][64 * wave + 4 * (lane & 3)];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const f16x8 bv = window_operand(base + 16 * nb);
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv, o[nb], 0, 0, 0);
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv, o[nb], 0, 0, 0);
      }
    }
    // merge weights of this lane's 4 heads: out = cg * global + cs * (window accumulator)
    float cg[4], cs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * (lane >> 4) + i;
      const float lg = sm.lse_g[h], ls = sm.lse_s[h];
      const float win = sm.unnorm * sm.inv_l[h];  // accumulator -> window result
      if (lg == -INFINITY) {
        cg[i] = 0.0f;
        cs[i] = win;
      } else {
        const float m = fmaxf(lg, ls);
        const float wg = expf(lg - m), ws = expf(ls - m);
        const float rn = 1.0f / (wg + ws);
        cg[i] = wg * rn;
        cs[i] = ws * rn * win;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int c = 256 * half + 64 * wave + 16 * nb + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * (lane >> 4) + i;
        a.out[((size_t)b * a.heads + h0 + h) * kLatent + c] = fmaf(cg[i], og[half][nb][i], cs[i] * o[nb][i]);
      }
    }
  }
  if (tid < kHg) {
    const float lg = sm.lse_g[tid], ls = sm.lse_s[tid];
    float r = ls;
    if (lg != -INFINITY) {
      const float m = fmaxf(lg, ls);
      r = m + logf(expf(lg - m) + expf(ls - m));
    }
    a.lse[(size_t)b * a.heads + h0 + tid] = r;
  }
}

// One wave per sequence: pack latent[b] into slot seq_lens[b] mod 128.
__global__ void __launch_bounds__(64) swa_append_kernel(uint8_t *codes, float *scales, const int32_t *pos,
                                                        const float *latent) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int p = pos[b];
  if (p < 0) return;
  const int slot = p % kWin;
  const float4 *src = reinterpret_cast<const float4 *>(latent + (size_t)b * kLatent + 8 * lane);
  const float4 u = src[0], v = src[1];
  const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float s = __fdiv_rn(amax, 448.0f);
  uint32_t w[2] = {0u, 0u};
  if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float qv = __fdiv_rn(x[i], s);
      const uint32_t c = e4m3_encode(fabsf(qv)) | ((__float_as_uint(x[i]) >> 31) << 7);
      w[i >> 2] |= c << (8 * (i & 3));
    }
  }
  reinterpret_cast<uint2 *>(codes + ((size_t)b * kWin + slot) * kLatent)[lane] = make_uint2(w[0], w[1]);
  if (lane == 0) scales[(size_t)b * kWin + slot] = s;
}

}  // namespace

hipError_t launch_swa_append(uint8_t *codes, float *scales, const int32_t *pos, int batch, const float *latent,
                             hipStream_t st) {
  if (batch == 0) return hipSuccess;
  swa_append_kernel<<<dim3(batch), dim3(64), 0, st>>>(codes, scales, pos, latent);
  return hipGetLastError();
}

hipError_t launch_swa_attn_merge(const uint8_t *codes, const float *scales, const int32_t *lens, int batch,
                                 const uint16_t *q, int heads, int qdim, float softmax_scale, float *out, float *lse,
                                 hipStream_t st) {
  if (batch == 0) return hipSuccess;
  SwaArgs a{codes, scales, lens, q, heads, qdim, softmax_scale * 1.4426950408889634f, out, lse};
  timer_before(kKernSwaAttn, st);
  swa_attn_kernel<<<dim3(batch, heads / kHg), dim3(256), 0, st>>>(a);
  timer_after(kKernSwaAttn, st);
  return hipGetLastError();
}

}  // namespace csa2
