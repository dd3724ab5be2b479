// Shared device helpers of libcsa2 (gfx950, wave64).
//
// FP4 format source: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section
// "FP4 KV cache": E2M1 elements, one E4M3 scale per 16 channels, no global
// scale; 448 x 6 = 2688 is the largest representable magnitude.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGroup = 16;        // channels per E4M3 scale
constexpr int kLatent = 512;      // latent channels
constexpr int kPage = 64;         // token slots per page
constexpr int kIdxDim = 64;       // indexer key width

// ---------------------------------------------------------------- E4M3FN
// Nearest E4M3FN code to a finite v >= 0, ties to the even code, saturating
// at 0x7E = 448.  Below 2^-6 the grid is uniform (k * 2^-9), so the code is
// the integer nearest to v * 2^9 (exact scaling, rintf rounds half to even).
// Above, the fp32 mantissa is rounded to 3 bits with the usual add-and-carry
// (a carry moves into the exponent field, which is the correct next code).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)rintf(v * 512.0f);  // 0..8 (8 == 0x08 == 2^-6)
  uint32_t b = __float_as_uint(v);
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // exponent + 7 - 127 = e - 120
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of an E4M3FN code (finite codes only: 0x7F / 0xFF never occur here).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------- E2M1
// Magnitude code of the E2M1 grid point nearest to |x| / s for s > 0.
// The decision points between neighbouring grid values are .25 .75 1.25 1.75
// 2.5 3.5 5 (times s; every product is exact in fp32).  On a tie the even
// code wins, which makes the comparison strict below an even code and
// inclusive below an odd one.  The code is the number of decision points
// passed; it is found by a three-level binary search (bit 2: 1.75, bit 1:
// 0.75 or 3.5, bit 0: .25 1.25 2.5 or 5), three compares instead of seven.
__device__ __forceinline__ uint32_t e2m1_magnitude(float ax, float s) {
  // the seven products do not depend on ax: callers packing a group share
  // them (the empty asm keeps the compiler from turning a select of two
  // products back into a product of a select, one multiply per value)
  float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
  float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
  asm("" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t4), "+v"(t5), "+v"(t6));
  const bool b2 = ax >= t3;
  const bool b1 = ax >= (b2 ? t5 : t1);
  const bool b0 = ax > (b2 ? (b1 ? t6 : t4) : (b1 ? t2 : t0));
  return 4u * b2 + 2u * b1 + (uint32_t)b0;
}

// Packs 16 consecutive channels: returns the E4M3 scale code and writes the
// 8 code bytes (channel 2j in the low nibble of byte j) into *lo / *hi words.
__device__ __forceinline__ uint32_t pack_group16(const float (&x)[16], uint32_t *w0, uint32_t *w1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float q = __fdiv_rn(amax, 6.0f);
  const uint32_t sc = e4m3_encode(q);
  const float s = e4m3_decode(sc);
  uint32_t words[2] = {0u, 0u};
  if (sc != 0u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t sign = (__float_as_uint(x[i]) >> 31) << 3;
      const uint32_t nib = sign | e2m1_magnitude(fabsf(x[i]), s);
      words[i >> 3] |= nib << (4 * (i & 7));
    }
  }
  *w0 = words[0];
  *w1 = words[1];
  return sc;
}

// E2M1 nibble -> float (exact).
__device__ __forceinline__ float e2m1_decode(uint32_t n) {
  const uint32_t c = n & 7u;
  // codes 2..7: 2^((c>>1)-1) * (1 + (c&1)/2) has fp32 bits (c << 22) + 0x3F000000
  uint32_t bits = c >= 2u ? (c << 22) + 0x3F000000u : (c == 1u ? 0x3F000000u : 0u);
  bits |= (n & 8u) << 28;
  return __uint_as_float(bits);
}

// Two E2M1 nibbles of byte `sel` of `word` -> two fp16 values times `s`
// (exact: at most 6 significant bits, magnitude in [2^-10, 2688]).  The
// hardware convert takes only the exponent of its scale operand, so it runs
// unscaled and the E4M3 scale is applied by one packed fp16 multiply.
template <int SEL>
__device__ __forceinline__ f16x2 deq2(uint32_t word, f16x2 s2) {
  f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
  return v * s2;
}

// 8 FP8 codes (two words) -> f16x8, exact.
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint2 w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 nibbles (one 32-bit word) -> f16x8 scaled by s.
__device__ __forceinline__ f16x8 deq8(uint32_t word, f16 s) {
  const f16x2 s2 = {s, s};
  const f16x2 a = deq2<0>(word, s2), b = deq2<1>(word, s2), c = deq2<2>(word, s2), d = deq2<3>(word, s2);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Order-preserving map of a finite float to uint32 (larger score -> larger
// key).  -0 is folded onto +0 first so equal scores give equal keys.  Key 0
// never comes from a finite float and marks "no item".
__device__ __forceinline__ uint32_t score_key(float s) {
  s = s + 0.0f;
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------- wave primitives
// Lane moves through DPP (data-parallel primitives of the VALU: no LDS round
// trip).  Controls: quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E,
// row_shr:n = 0x110 + n, row_mirror = 0x140, row_half_mirror = 0x141,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.  Lanes with no source read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Sum over the aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float group8_sum(float s) {
  s += dpp_f32<0xB1>(s);
  s += dpp_f32<0x4E>(s);
  s += dpp_f32<0x141>(s);
  return s;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp_u32<0x111>(v);
  v += dpp_u32<0x112>(v);
  v += dpp_u32<0x114>(v);
  v += dpp_u32<0x118>(v);
  v += dpp_u32<0x142, 0xA>(v);
  v += dpp_u32<0x143, 0xC>(v);
  return v;
}

// Inclusive prefix maximum (unsigned) over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_max(uint32_t v) {
  v = max(v, dpp_u32<0x111>(v));
  v = max(v, dpp_u32<0x112>(v));
  v = max(v, dpp_u32<0x114>(v));
  v = max(v, dpp_u32<0x118>(v));
  v = max(v, dpp_u32<0x142, 0xA>(v));
  v = max(v, dpp_u32<0x143, 0xC>(v));
  return v;
}

// Value of lane 63 (e.g. the total after an inclusive sum), uniform.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 63); }

}  // namespace csa2
