// Sparse FP4 decode attention over the selected entries of a paged cache.
//
// Sources: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "CSA2"
// (one small latent shared by all heads; each layer attends over its top-K
// selected entries) and section "FP4 KV cache" (the cache is dequantized
// before attention); ingu627 asymmetric-serving blog, section 2 (64 heads,
// one KV head).  For each sequence b and head h over the valid selected set S:
//   logit_s = scale * (q[h,:512] . c_s + q[h,512:] . rope_s)
//   out[h]  = sum_s softmax(logit)_s c_s,   lse[h] = log sum_s exp(logit_s)
// with c_s the dequantized 512-channel latent (K = V).
//
// Design (ours):
//   * One workgroup (4 waves) serves up to 64 heads of one sequence, so each
//     dequantized entry feeds every head: QK^T and PV are MFMA contractions
//     with M = heads (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//   * Entries are processed in tiles of 32.  A tile's FP4 codes are gathered
//     straight into registers (8 lanes per 256-byte row), dequantized with the
//     hardware E2M1 -> fp16 convert plus one packed multiply by the E4M3 scale
//     (exact), and written once to LDS, row-major.  QK^T reads its operand
//     (channels contiguous) with 16-byte loads; PV reads its operand (entries
//     contiguous) with gfx950's transposing LDS loads, so no transposed copy
//     of the tile is made.
//   * Online softmax in fp32 (exp2 domain) against a reference max that
//     moves only when a logit exceeds it by more than 8 (so most tiles skip
//     rescaling the accumulators).  P enters the PV contraction as
//     fp16 hi + lo parts (two MFMAs), which keeps the output within ~1e-5
//     relative of an fp32 P; a single fp16 P is not accurate enough for
//     latents with x20 outlier channels.
//   * Split-K over entries across workgroups for small batches; partial
//     (m, l, O) are merged by an lse-weighted combine kernel (one wave per
//     256 channels when there are few splits, one workgroup per 64 channels
//     that loads all splits at once when there are many).
//   * The sliding-window branch (sections "KV bottleneck" and "FP4 KV
//     cache": a local window of 128 FP8 entries beside the global selection;
//     merged as one softmax over the union of both entry sets, this library's
//     reading) can ride along: its 128 ring slots are four more split
//     workgroups of one 32-entry tile each.  Their tile holds the E4M3 codes
//     as fp16 (exact) with a zero rope part (window keys have none); the
//     per-token fp32 scale multiplies the logit, and P times that scale
//     (normalized by a power of two into [1, 2) over the tile, undone on the
//     partial) enters PV, so the combine merges window and global partials
//     alike.  The current token's window entry can be appended in the same
//     launch: the window workgroups of the tile holding its slot pack it to
//     FP8 (the same rounding as the standalone append) into LDS and use it
//     from there, and the first head group's one writes it to the ring.
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int kT = 32;                 // entries per tile
constexpr int kQkLd = kLatent + 64 + 8;  // row-major tile row (f16): 512 latent + 64 rope + pad
constexpr int kPLd = kT + 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 32;         // split-K workgroups per (sequence, head group)
constexpr int kSlotCap = 2048;         // entries one workgroup resolves up front
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
constexpr int kWinSlots = 128;          // sliding-window ring slots per sequence
constexpr int kWinSplits = kWinSlots / kT;  // window tiles = extra split workgroups

struct AttnArgs {
  KvLayerDev L;
  SeqsDev S;
  const uint16_t *q;      // [B][H][512 + rope]
  const int32_t *idx;     // [B][K]
  int heads;              // H
  int top_k;
  int splits;             // workgroups per (b, head group) along the selected entries
  int parts;              // partials per (b, head): splits, plus kWinSplits with the window
  int tiles_per_split;
  uint8_t *win_codes;        // [B][128][512] E4M3 window entries, or null
  float *win_scales;         // [B][128] per-token scales
  const float *win_latent;   // [B][512] the current token's window entry to append first, or null
  float scale_log2;       // softmax scale * log2(e)
  float *out;             // [B][H][512]  (splits == 1)
  float *lse;             // [B][H] or null
  float *part_o;          // [B][H][parts][512]  (parts > 1)
  float *part_ml;         // [B][H][parts][2]
};

template <int MT>
struct __attribute__((aligned(16))) Smem {  // 16-byte aligned rows: every tile access is a 128-bit LDS op
  __attribute__((aligned(16))) f16 cq[3][kT][kQkLd];   // row-major dequantized tiles (+ rope), used in turn
  float s[2][16 * MT][kT + 1];   // logits of the tile (two k-halves when 16 heads; padded rows)
  __attribute__((aligned(16))) f16 p_hi[16 * MT][kPLd];
  __attribute__((aligned(16))) f16 p_lo[16 * MT][kPLd];
  float m_run[16 * MT], l_run[16 * MT], alpha[16 * MT];
  uint32_t slot[kSlotCap];       // physical rows of this workgroup's entries (kNoSlot: skipped)
  float wts[kT], wp[kT];         // window tile: token scales, and times the P normalization
  float unnorm;                  // window tile: the P normalization, inverted
  float wamax[4];                // appended window entry: per-wave amax
  __attribute__((aligned(16))) uint8_t newc[kLatent];  // appended window entry: E4M3 codes
};

__device__ __forceinline__ f16x8 lds_f16x8(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// PV operand (B of v_mfma_f32_16x16x32_f16, k = entries, n = channels) read
// straight from the row-major tile with two transposing LDS loads.  Within a
// group of 16 lanes, ds_read_b64_tr_b16 hands lane i element i % 4 of the
// 8-byte chunks read by lanes 4 e + i / 4 (e = 0..3).  Lane L of k-group
// g = L / 16 therefore points at row 8 g + (L / 4) % 4 (+ 4 for the second
// load), channels n0 + 4 (L % 4) .. + 3, and receives rows 8 g .. 8 g + 7 of
// channel n0 + L % 16.  p: that lane's first-load address.
__device__ __forceinline__ f16x8 pv_operand(const f16 *p) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * kQkLd));
  const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(f16x8, ab);
}

__device__ __forceinline__ f16x8 bf16x8_to_f16x8(uint4 v) {
  f16x8 r;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (f16)__uint_as_float(w[i] << 16);
    r[2 * i + 1] = (f16)__uint_as_float(w[i] & 0xFFFF0000u);
  }
  return r;
}

// Reductions over aligned groups of G = 4, 8 or 16 lanes (DPP, every lane gets the result).
template <int G>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);
  return v;
}

// Raw FP4 row fragment of one entry: 64 channels of codes, their 4 scales and
// (with rope) 8 rope values.
struct Raw {
  uint4 c0, c1, rp;
  uint32_t sc4;
  bool valid;
};

template <int MT, bool ROPE>
__global__ void __launch_bounds__(256) sparse_attn_kernel(AttnArgs a) {
  constexpr int HG = 16 * MT;                  // heads in this workgroup
  constexpr int QW = kLatent + (ROPE ? 64 : 0);  // q row width
  constexpr int KS = QW / 32;                  // 16 or 18 k-steps of 32 channels
  __shared__ Smem<MT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int h0 = hg * HG;
  const int n = min(max(a.S.seq_lens[b], 0), a.S.max_len);
  // workgroups past the selection's splits take window tile split - splits:
  // ring slots 32 wt .. 32 wt + 31, valid below min(seq_len, 128)
  const bool win = split >= a.splits;
  const int wt = split - a.splits;
  const int nwin = min(max(a.S.seq_lens[b], 0), kWinSlots);
  const int s_new = nwin > 0 ? (a.S.seq_lens[b] - 1) % kWinSlots : -1;  // the current token's slot
  const bool pack_new = win && a.win_latent != nullptr && s_new >= 0 && s_new / kT == wt;

  const int n_tiles_all = (a.top_k + kT - 1) / kT;
  const int tile_begin = win ? 0 : split * a.tiles_per_split;
  const int tile_end = win ? (nwin > kT * wt ? 1 : 0) : min(tile_begin + a.tiles_per_split, n_tiles_all);
  const int e_begin = tile_begin * kT;
  // <= kSlotCap (host-chosen splits)
  const int e_count = win ? kT : max(0, min(tile_end * kT, a.top_k) - e_begin);
  const int32_t *idx_row = a.idx + (size_t)b * a.top_k;

  // ---- QK^T work of this wave: one M-tile (16 heads) and 1 or 2 N-tiles of 16 entries
  // (16 heads: every wave takes one N-tile and half of the k-steps; the two
  // halves of a logit are added when the softmax reads them)
  constexpr int QKS = MT == 1 ? KS / 2 : KS;  // k-steps per wave
  int qk_mt, qk_nt0, qk_ntn, qk_half;
  if constexpr (MT == 4) { qk_mt = wave; qk_nt0 = 0; qk_ntn = 2; qk_half = 0; }
  else if constexpr (MT == 2) { qk_mt = wave >> 1; qk_nt0 = wave & 1; qk_ntn = 1; qk_half = 0; }
  else { qk_mt = 0; qk_nt0 = wave & 1; qk_ntn = 1; qk_half = wave >> 1; }
  const int qk_k0 = qk_half * QKS;

  // ---- entry indices of this workgroup, then their physical rows (two dependent
  // reads for all entries at once; the q loads below overlap them)
  int pos[kSlotCap / 256];
#pragma unroll
  for (int j = 0; j < kSlotCap / 256; ++j) pos[j] = -1;
  if (!win) {
#pragma unroll
    for (int j = 0; j < kSlotCap / 256; ++j) {
      if (256 * j >= e_count) break;  // uniform: rounds past this workgroup's entries are not read
      const int i = 256 * j + tid;
      const int p = idx_row[min(e_begin + i, a.top_k - 1)];  // clamped read, masked below
      pos[j] = i < e_count ? p : -1;
    }
  }

  // q fragments (A operand): head 16*qk_mt + lane%16, channels 32*(qk_k0 + ks) + 8*(lane/16) .. +7
  f16x8 qf[QKS];
  {
    const uint16_t *qrow =
        a.q + ((size_t)b * a.heads + h0 + 16 * qk_mt + (lane & 15)) * QW + 32 * qk_k0 + 8 * (lane >> 4);
    uint4 raw[QKS];
#pragma unroll
    for (int ks = 0; ks < QKS; ++ks) raw[ks] = *reinterpret_cast<const uint4 *>(qrow + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < QKS; ++ks) qf[ks] = bf16x8_to_f16x8(raw[ks]);
  }

  if (!win) {
    int blk[kSlotCap / 256];
#pragma unroll
    for (int j = 0; j < kSlotCap / 256; ++j) {
      if (256 * j >= e_count) break;  // (slots past e_count are never read)
      const int p = pos[j];
      const bool ok = p >= 0 && p < n && p / kPage < a.S.max_blocks;
      // clamped read, masked below (a table without columns maps nothing)
      blk[j] = a.S.max_blocks > 0 ? a.S.block_table[(size_t)b * a.S.max_blocks + (ok ? p / kPage : 0)] : -1;
      pos[j] = ok ? p : -1;
    }
#pragma unroll
    for (int j = 0; j < kSlotCap / 256; ++j) {
      if (256 * j >= e_count) break;
      const int i = 256 * j + tid;
      const bool ok = pos[j] >= 0 && blk[j] >= 0 && blk[j] < a.L.num_blocks;
      sm.slot[i] = ok ? (uint32_t)blk[j] * kPage + (uint32_t)(pos[j] % kPage) : kNoSlot;
    }
  } else {
    // appending the current token's entry (slot (n - 1) mod 128) when this tile holds it: FP8 pack with
    // s = amax / 448, code = E4M3(x / s); each thread packs channels 2 tid, 2 tid + 1
    float snew = 0.0f;
    if (pack_new) {
      const float2 x = reinterpret_cast<const float2 *>(a.win_latent + (size_t)b * kLatent)[tid];
      float m = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) sm.wamax[wave] = m;
      __syncthreads();  // uniform: the whole workgroup packs
      const float amax = fmaxf(fmaxf(sm.wamax[0], sm.wamax[1]), fmaxf(sm.wamax[2], sm.wamax[3]));
      snew = __fdiv_rn(amax, 448.0f);
      uint32_t c0 = 0u, c1 = 0u;
      if (snew > 0.0f) {
        c0 = e4m3_encode(fabsf(__fdiv_rn(x.x, snew))) | ((__float_as_uint(x.x) >> 31) << 7);
        c1 = e4m3_encode(fabsf(__fdiv_rn(x.y, snew))) | ((__float_as_uint(x.y) >> 31) << 7);
      }
      const uint16_t c = (uint16_t)(c0 | (c1 << 8));
      reinterpret_cast<uint16_t *>(sm.newc)[tid] = c;
      if (hg == 0) {  // one head group writes the ring
        reinterpret_cast<uint16_t *>(a.win_codes + ((size_t)b * kWinSlots + s_new) * kLatent)[tid] = c;
        if (tid == 0) a.win_scales[(size_t)b * kWinSlots + s_new] = snew;
      }
    }
    if (tid < kT) {
      // window tile: ring slots, token scales, and a power of two that brings the
      // tile's largest token scale into [1, 2) (P times the scale stays in fp16's
      // normal range)
      const int s = kT * wt + tid;
      const bool ok = s < nwin;
      sm.slot[tid] = ok ? (uint32_t)s : kNoSlot;
      const float ts = !ok ? 0.0f : (pack_new && s == s_new) ? snew : a.win_scales[(size_t)b * kWinSlots + s];
      float mx = ts;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float norm = mx > 0.0f ? __uint_as_float((254u - ((__float_as_uint(mx) >> 23) & 0xFFu)) << 23) : 1.0f;
      sm.wts[tid] = ts;
      sm.wp[tid] = ts * norm;
      if (tid == 0) sm.unnorm = 1.0f / norm;
    }
  }

  // ---- PV accumulators: wave owns channels [128*wave, 128*wave+128) for all HG heads
  f32x4 acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // slot[] is complete

  // gather of one tile: thread -> entry tile_entry, channel block tile_block
  // (channels 64 tile_block .. + 63).  A wave covers 8 entries; its
  // lanes 16 i .. 16 i + 15 take the 8 entries at blocks 2 i and 2 i + 1, so
  // each 16-byte LDS store of the dequantized tile (row stride 73 x 16 bytes)
  // lands the 16 lanes on 16 different bank groups.  Every load is issued
  // unconditionally (a skipped entry reads row 0 and is zeroed when
  // dequantized; an empty pool never launches a tile).
  const int tile_entry = (tid & 7) + 8 * wave, tile_block = (lane >> 3) & 7;
  auto load_raw = [&](int tile, Raw &r) {
    const int e = tile_entry, cb = tile_block;
    const int li = tile * kT + e - e_begin;
    const uint32_t slot = li < e_count ? sm.slot[li] : kNoSlot;
    const size_t rs = slot == kNoSlot ? 0 : slot;
    const uint4 *cp = reinterpret_cast<const uint4 *>(a.L.codes + rs * (kLatent / 2) + 32 * cb);
    r.c0 = cp[0];
    r.c1 = cp[1];
    r.sc4 = *reinterpret_cast<const uint32_t *>(a.L.scales + rs * (kLatent / kGroup) + 4 * cb);
    if constexpr (ROPE) r.rp = *reinterpret_cast<const uint4 *>(a.L.rope + rs * 64 + 8 * cb);
    r.valid = slot != kNoSlot;
  };

  // dequantize one tile's row fragments into a row-major tile buffer
  // (branch-free: a skipped entry is masked to scale 0 and rope 0, so its
  // channels are all zero; the four E4M3 scales go through the hardware fp8
  // convert, exact in fp16)
  auto dequant = [&](const Raw &r, f16 (*cq)[kQkLd]) {
    const int e = tile_entry, cb = tile_block;
    const uint32_t vmask = 0u - (uint32_t)r.valid;
    const uint32_t words[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    const uint32_t sc4 = r.sc4 & vmask;
    const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc4, 1.0f, false);  // scale bytes 0, 1
    const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc4, 1.0f, true);   // scale bytes 2, 3
    const f16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
    for (int wi = 0; wi < 8; ++wi)
      *reinterpret_cast<f16x8 *>(&cq[e][64 * cb + 8 * wi]) = deq8(words[wi], sc[wi >> 1]);
    if constexpr (ROPE) {
      const uint4 rp = make_uint4(r.rp.x & vmask, r.rp.y & vmask, r.rp.z & vmask, r.rp.w & vmask);
      *reinterpret_cast<f16x8 *>(&cq[e][kLatent + 8 * cb]) = bf16x8_to_f16x8(rp);
    }
  };

  // online-softmax state: thread -> head tid / TPH, entries (tid % TPH) * EPT ..
  // + EPT - 1 of a tile; the TPH threads of a head keep the same running max
  // and sum in registers
  constexpr int TPH = 256 / HG;   // threads per head (4, 8 or 16)
  constexpr int EPT = kT / TPH;   // entries per thread (8, 4 or 2)
  const int sm_h = tid / TPH, sm_part = tid % TPH;
  float m_run = -INFINITY, l_run = 0.f;

  // One tile from buffer cq, with the next tile's dequantization into cq_next
  // (three buffers in turn) in the same phase.  Two barriers per tile: the
  // buffer a phase writes was last read two barriers earlier.
  auto step = [&](int tile, f16 (*cq)[kQkLd], const Raw *next, f16 (*cq_next)[kQkLd]) {
    // 1. logits S = scale * Q C^T  (this wave's M-tile, 1 or 2 N-tiles)
    for (int j = 0; j < qk_ntn; ++j) {
      const int nt = qk_nt0 + j;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const f16 *brow = &cq[16 * nt + (lane & 15)][32 * qk_k0 + 8 * (lane >> 4)];
      f16x8 bq[QKS];  // B fragments read 4 k-steps ahead of the MFMA that consumes them
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bq[ks] = lds_f16x8(brow + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks) {
        if (ks + 4 < QKS) bq[ks + 4] = lds_f16x8(brow + 32 * (ks + 4));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[ks], bq[ks], sacc, 0, 0, 0);
      }
      // lane holds S[head 16*mt + 4*(lane/16) + r][entry 16*nt + lane%16] (this wave's k-half)
      const int ent = 16 * nt + (lane & 15);
      const int li = tile * kT + ent - e_begin;
      const bool valid = qk_half == 1 || (li < e_count && sm.slot[li] != kNoSlot);  // masked once
      float es = a.scale_log2;
      if (win) es *= sm.wts[ent];  // window entries: the token scale of the E4M3 codes
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        sm.s[qk_half][16 * qk_mt + 4 * (lane >> 4) + rr][ent] = valid ? sacc[rr] * es : -INFINITY;
    }
    if (next != nullptr) dequant(*next, cq_next);
    __syncthreads();
    // 2. online softmax
    {
      float v[EPT];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        v[i] = sm.s[0][sm_h][sm_part * EPT + i];
        if constexpr (MT == 1) v[i] += sm.s[1][sm_h][sm_part * EPT + i];
        mx = fmaxf(mx, v[i]);
      }
      mx = group_max<TPH>(mx);
      // The reference m_run moves only when a logit exceeds it by more than
      // 2^8 (in the exp2 domain): weights stay below 2^8, O and l are left
      // unscaled on most tiles, and O / l is the same ratio.
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float pv = (m_new == -INFINITY) ? 0.f : exp2f(v[i] - m_new);
        sum += pv;
        const float pw = win ? pv * sm.wp[sm_part * EPT + i] : pv;  // window: P times the token scale
        const f16 ph = (f16)pw;
        const f16 pl = (f16)(pw - (float)ph);
        sm.p_hi[sm_h][sm_part * EPT + i] = ph;
        sm.p_lo[sm_h][sm_part * EPT + i] = pl;
      }
      sum = group_sum<TPH>(sum);
      // (from an empty state O and l are zero: no rescaling either)
      const float al = (m_new == m_run || m_run == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      l_run = l_run * al + sum;
      m_run = m_new;
      if (sm_part == 0) sm.alpha[sm_h] = al;
    }
    __syncthreads();
    // 3. O = alpha * O + P V  (wave: channels 128*wave .. +127, all heads)
    {
      float al[MT][4];
      bool rescale = false;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          al[mt][rr] = sm.alpha[16 * mt + 4 * (lane >> 4) + rr];
          rescale |= al[mt][rr] != 1.f;
        }
      if (__ballot(rescale)) {  // the accumulators live in AGPRs: scale only when a reference moved
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[mt][nt][rr] *= al[mt][rr];
      }
      f16x8 ph[MT], pl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ph[mt] = lds_f16x8(&sm.p_hi[16 * mt + (lane & 15)][8 * (lane >> 4)]);
        pl[mt] = lds_f16x8(&sm.p_lo[16 * mt + (lane & 15)][8 * (lane >> 4)]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const f16x8 bv = pv_operand(&cq[8 * (lane >> 4) + ((lane >> 2) & 3)][128 * wave + 16 * nt + 4 * (lane & 3)]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[mt], bv, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[mt], bv, acc[mt][nt], 0, 0, 0);
        }
      }
    }
  };

  // ---- tiles: three register sets of raw rows (each tile's loads are issued
  // three tiles ahead; loads past the last tile re-read the last tile) and
  // three tile buffers, so the unrolled loop keeps both in step
  if (win) {
    if (tile_begin < tile_end) {
      // the window tile: thread -> entry tile_entry, channels 64 tile_block .. + 63
      // (64 E4M3 bytes), converted to fp16 (exact); skipped slots and the rope
      // part are zero
      const uint32_t slot = sm.slot[tile_entry];
      const uint4 *cp = pack_new && slot == (uint32_t)s_new  // the appended entry, from LDS
                            ? reinterpret_cast<const uint4 *>(sm.newc + 64 * tile_block)
                            : reinterpret_cast<const uint4 *>(a.win_codes +
                                                              ((size_t)b * kWinSlots + (slot == kNoSlot ? 0 : slot)) *
                                                                  kLatent +
                                                              64 * tile_block);
      uint4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = cp[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 lo = fp8x8_to_f16(make_uint2(w[i].x, w[i].y));
        f16x8 hi = fp8x8_to_f16(make_uint2(w[i].z, w[i].w));
        if (slot == kNoSlot) lo = hi = f16x8{};
        *reinterpret_cast<f16x8 *>(&sm.cq[0][tile_entry][64 * tile_block + 16 * i]) = lo;
        *reinterpret_cast<f16x8 *>(&sm.cq[0][tile_entry][64 * tile_block + 16 * i + 8]) = hi;
      }
      if constexpr (ROPE) *reinterpret_cast<f16x8 *>(&sm.cq[0][tile_entry][kLatent + 8 * tile_block]) = f16x8{};
      __syncthreads();
      step(0, sm.cq[0], nullptr, sm.cq[1]);
    }
  } else if (tile_begin < tile_end && a.L.num_blocks > 0) {
    const int last = tile_end - 1;
    Raw ra, rb, rc;
    load_raw(tile_begin, ra);
    load_raw(min(tile_begin + 1, last), rb);
    load_raw(min(tile_begin + 2, last), rc);
    dequant(ra, sm.cq[0]);
    load_raw(min(tile_begin + 3, last), ra);
    __syncthreads();
    for (int tile = tile_begin; tile < tile_end; tile += 3) {
      step(tile, sm.cq[0], tile + 1 < tile_end ? &rb : nullptr, sm.cq[1]);
      load_raw(min(tile + 4, last), rb);
      if (tile + 1 < tile_end) {
        step(tile + 1, sm.cq[1], tile + 2 < tile_end ? &rc : nullptr, sm.cq[2]);
        load_raw(min(tile + 5, last), rc);
      }
      if (tile + 2 < tile_end) {
        step(tile + 2, sm.cq[2], tile + 3 < tile_end ? &ra : nullptr, sm.cq[0]);
        load_raw(min(tile + 6, last), ra);
      }
    }
  }
  if (sm_part == 0) {
    sm.m_run[sm_h] = m_run;
    sm.l_run[sm_h] = l_run;
  }
  __syncthreads();

  // ---- write the result straight from the accumulators (PV column = channel):
  // final rows when unsplit, else a partial for the combine; the 16 lanes of a
  // row group write 64 contiguous bytes.
  const bool final_out = a.parts == 1;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 16 * mt + 4 * (lane >> 4) + r;
      const size_t h = (size_t)b * a.heads + h0 + hl;
      float sc = win ? sm.unnorm : 1.0f;
      float *dst = a.part_o + (h * a.parts + split) * kLatent;
      if (final_out) {
        const float l = sm.l_run[hl];
        sc = l > 0.f ? 1.0f / l : 0.f;
        dst = a.out + h * kLatent;
      }
      dst += 128 * wave + (lane & 15);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) dst[16 * nt] = acc[mt][nt][r] * sc;
    }
  if (final_out) {
    if (a.lse != nullptr && tid < HG) {
      const float l = sm.l_run[tid];
      a.lse[(size_t)b * a.heads + h0 + tid] = l > 0.f ? (sm.m_run[tid] + log2f(l)) / kLog2e : -INFINITY;
    }
  } else if (tid < HG) {
    float *ml = a.part_ml + (((size_t)b * a.heads + h0 + tid) * a.parts + split) * 2;
    ml[0] = sm.m_run[tid];
    ml[1] = sm.l_run[tid];
  }
}

// Merges the splits' partials: workgroup (b*H + h, half) of one full wave
// covers 256 channels of one head, one float4 per thread.  Splits are read 8
// at a time (all loads of a chunk issued together) and merged online.
constexpr int kCombineThreads = 64;
__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int splits,
                                                          float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kChunk = 8;  // the launch sends this kernel at most 8 splits (more go to the wide merge)
  const int bh = blockIdx.x, quarter = blockIdx.y;  // quarter: which kCombineThreads float4s
  const int tid = threadIdx.x;
  const int c4 = kCombineThreads * quarter + tid;  // float4 index within the 512 channels
  const float2 *ml = reinterpret_cast<const float2 *>(part_ml + (size_t)bh * splits * 2);
  float m = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += kChunk) {
    // unconditional loads (clamped split index); splits past the end and empty
    // splits (m = -inf, l = 0, O = 0) get weight 0
    float2 mls[kChunk];
    float4 po[kChunk];
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const int sc = s0 + s < splits ? s0 + s : s0;
      mls[s] = ml[sc];
      po[s] = reinterpret_cast<const float4 *>(part_o + ((size_t)bh * splits + sc) * kLatent)[c4];
    }
    float mc = m;
#pragma unroll
    for (int s = 0; s < kChunk; ++s)
      if (s0 + s < splits) mc = fmaxf(mc, mls[s].x);
    const float r = (m == -INFINITY) ? 0.f : exp2f(m - mc);  // rescale what is merged so far
    l *= r;
    o.x *= r;
    o.y *= r;
    o.z *= r;
    o.w *= r;
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const float w = (s0 + s < splits && mls[s].x != -INFINITY) ? exp2f(mls[s].x - mc) : 0.f;
      l += w * mls[s].y;
      o.x += w * po[s].x;
      o.y += w * po[s].y;
      o.z += w * po[s].z;
      o.w += w * po[s].w;
    }
    m = mc;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  reinterpret_cast<float4 *>(out + (size_t)bh * kLatent)[c4] = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (lse != nullptr && quarter == 0 && tid == 0) lse[bh] = l > 0.f ? (m + log2f(l)) / kLog2e : -INFINITY;
}

// The same merge for many splits (batch-1 decode): workgroup (b*H + h, q)
// covers 64 channels of one head with 256 threads, 16 float4 columns x 16
// split groups (splits g, g + 16, .. : PER each), then one merge of the 16
// groups through LDS: one round of loads instead of a long chain per thread.
constexpr int kWideThreads = 256;
constexpr int kWideCols = 16;  // float4 columns per workgroup
constexpr int kWideMaxPer = 3;  // splits per thread at most
template <int kWidePer>
__global__ void __launch_bounds__(kWideThreads) attn_combine_wide_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int splits,
                                                          float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kGroups = kWideThreads / kWideCols;  // 16
  static_assert(kMaxSplits + kWinSplits <= kWideMaxPer * kGroups, "splits per thread");
  __shared__ float4 so[kGroups][kWideCols];
  __shared__ float gm[kGroups], sl[kGroups];
  const int bh = blockIdx.x, q = blockIdx.y;
  const int tid = threadIdx.x, col = tid % kWideCols, g = tid / kWideCols;
  const int c4 = kWideCols * q + col;
  const float2 *ml = reinterpret_cast<const float2 *>(part_ml + (size_t)bh * splits * 2);
  const float4 *po = reinterpret_cast<const float4 *>(part_o + (size_t)bh * splits * kLatent);
  float2 a[kWidePer];
  float4 p[kWidePer];
#pragma unroll
  for (int j = 0; j < kWidePer; ++j) {  // unconditional loads (clamped split index), masked below
    const int s = g + kGroups * j;
    const int sc = s < splits ? s : 0;
    a[j] = ml[sc];
    p[j] = po[(size_t)sc * (kLatent / 4) + c4];
  }
  float mj[kWidePer];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kWidePer; ++j) {
    mj[j] = g + kGroups * j < splits ? a[j].x : -INFINITY;
    m = fmaxf(m, mj[j]);
  }
  float l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kWidePer; ++j) {
    const float w = mj[j] == -INFINITY ? 0.f : exp2f(mj[j] - m);  // empty splits: m = -inf, l = 0, O = 0
    l += w * a[j].y;
    o.x += w * p[j].x;
    o.y += w * p[j].y;
    o.z += w * p[j].z;
    o.w += w * p[j].w;
  }
  so[g][col] = o;
  if (col == 0) {
    gm[g] = m;
    sl[g] = l;
  }
  __syncthreads();
  if (tid < kWideCols) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGroups; ++i) mx = fmaxf(mx, gm[i]);
    float lt = 0.f;
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const float w = gm[i] == -INFINITY ? 0.f : exp2f(gm[i] - mx);
      const float4 x = so[i][tid];
      lt += w * sl[i];
      r.x += w * x.x;
      r.y += w * x.y;
      r.z += w * x.z;
      r.w += w * x.w;
    }
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    reinterpret_cast<float4 *>(out + (size_t)bh * kLatent)[kWideCols * q + tid] =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    if (lse != nullptr && q == 0 && tid == 0) lse[bh] = lt > 0.f ? (mx + log2f(lt)) / kLog2e : -INFINITY;
  }
}

// Heads per workgroup.  64 shares each dequantized tile among the most heads;
// when that leaves the chip short of workgroups (small batches) 16 heads per
// workgroup give 4x the workgroups, each with a quarter of the MFMA work per
// tile (the tile is then dequantized once per head group, from L2).
int heads_per_group(int batch, int heads) {
  if (heads % 64 == 0 && (int64_t)batch * (heads / 64) >= 32) return 64;
  return 16;
}

int choose_splits(int batch, int heads, int top_k) {
  const int groups = batch * (heads / heads_per_group(batch, heads));
  const int tiles = (top_k + kT - 1) / kT;
  int splits = (256 + groups - 1) / groups;  // about one workgroup per CU
  if (splits > tiles) splits = tiles;
  if (splits > kMaxSplits) splits = kMaxSplits;
  const int min_splits = (tiles * kT + kSlotCap - 1) / kSlotCap;  // a workgroup resolves at most kSlotCap entries
  if (splits < min_splits) splits = min_splits;
  if (splits < 1) splits = 1;
  return splits;
}

}  // namespace

size_t attn_workspace_bytes(int batch, int heads, int top_k, bool window) {
  const int parts = choose_splits(batch, heads, top_k) + (window ? kWinSplits : 0);
  if (parts == 1) return 256;
  const size_t o = (size_t)batch * heads * parts * kLatent * sizeof(float);
  const size_t ml = (size_t)batch * heads * parts * 2 * sizeof(float);
  return ((o + 255) & ~(size_t)255) + ((ml + 255) & ~(size_t)255);
}

hipError_t launch_sparse_attn(const KvLayerDev &L, const SeqsDev &S, const uint16_t *q, int heads,
                              const int32_t *indices, int top_k, float scale, uint8_t *win_codes,
                              float *win_scales, const float *win_latent, float *out, float *lse, void *ws,
                              hipStream_t st) {
  if (S.batch == 0) return hipSuccess;
  const bool window = win_codes != nullptr;
  const int hgsz = heads_per_group(S.batch, heads);
  const int splits = choose_splits(S.batch, heads, top_k);
  const int parts = splits + (window ? kWinSplits : 0);
  const int tiles = (top_k + kT - 1) / kT;
  AttnArgs a;
  a.L = L;
  a.S = S;
  a.q = q;
  a.idx = indices;
  a.heads = heads;
  a.top_k = top_k;
  a.splits = splits;
  a.parts = parts;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  a.win_codes = win_codes;
  a.win_scales = win_scales;
  a.win_latent = win_latent;
  a.scale_log2 = scale * kLog2e;
  a.out = out;
  a.lse = lse;
  const size_t o_bytes = (size_t)S.batch * heads * parts * kLatent * sizeof(float);
  a.part_o = static_cast<float *>(ws);
  a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((o_bytes + 255) & ~(size_t)255));
  const dim3 grid(parts, heads / hgsz, S.batch);
  timer_before(kKernSparseAttn, st);
  const bool rope = L.rope_dim != 0;
  if (hgsz == 64) {
    if (rope) sparse_attn_kernel<4, true><<<grid, dim3(256), 0, st>>>(a);
    else sparse_attn_kernel<4, false><<<grid, dim3(256), 0, st>>>(a);
  } else {
    if (rope) sparse_attn_kernel<1, true><<<grid, dim3(256), 0, st>>>(a);
    else sparse_attn_kernel<1, false><<<grid, dim3(256), 0, st>>>(a);
  }
  timer_after(kKernSparseAttn, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts == 1) return e;
  timer_before(kKernAttnCombine, st);
  const dim3 wide_grid(S.batch * heads, kLatent / 4 / kWideCols);
  if (parts > 32)
    attn_combine_wide_kernel<3><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, out, lse);
  else if (parts > 16)
    attn_combine_wide_kernel<2><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, out, lse);
  else if (parts > 8)
    attn_combine_wide_kernel<1><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, out, lse);
  else
    attn_combine_kernel<<<dim3(S.batch * heads, kLatent / 4 / kCombineThreads), dim3(kCombineThreads), 0, st>>>(
        a.part_o, a.part_ml, parts, out, lse);
  timer_after(kKernAttnCombine, st);
  return hipGetLastError();
}

}  // namespace csa2
