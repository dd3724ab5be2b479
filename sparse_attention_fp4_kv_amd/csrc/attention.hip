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
//   * One workgroup (8 waves, two per SIMD) serves 16, 32 or 64 heads of one
//     sequence, so each dequantized entry feeds all of them: QK^T and PV are
//     MFMA contractions with M = heads (v_mfma_f32_16x16x32_f16, fp32
//     accumulation).  QK^T splits each 16 x 16 logit tile's 512 (+64)
//     channels over 2 or 4 waves (partial logits added in the softmax), with
//     2 or 4 independent accumulator chains per wave; PV gives each wave 64
//     output channels of every head.
//   * Entries are processed in tiles of 32.  A tile's FP4 codes are gathered
//     straight into registers (16 bytes per lane, 4 lanes per 64 contiguous
//     bytes of a row), dequantized with the hardware E2M1 -> fp16 convert
//     times the E4M3 scale (exact), and written once to LDS, row-major, each
//     16-byte store of a half-wave on 16 different bank groups.  QK^T reads
//     its operand (channels contiguous) with 16-byte loads; PV reads its
//     operand (entries contiguous) with gfx950's transposing LDS loads, so no
//     transposed copy of the tile is made.
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
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace csa2 {

// Scratch of the allocation-free attention entry point: the split partials of
// one launch live here instead of in a caller workspace.  Every device the
// library runs on holds its own copy until the process ends; its address is
// resolved once per device (hipGetSymbolAddress) and only that address is
// handed to kernels.
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

hipError_t attn_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}


namespace {

constexpr int kT = 32;                 // entries per tile
constexpr int kThreads = 512;          // 8 waves per workgroup (two per SIMD)
constexpr int kWaves = kThreads / 64;
constexpr int kPLd = kT + 8;
// waves splitting the k-steps (channels) of one 16 x 16 logit tile: with 16
// heads the 8 waves take 2 N-tiles x 4 k-parts, else M-tiles x N-tiles x 2
template <int MT>
constexpr int kKParts = MT == 1 ? 4 : 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 32;         // split-K workgroups per (sequence, head group)
constexpr int kSlotCap = 2048;         // entries one workgroup resolves up front
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
constexpr int kWinSlots = 128;          // sliding-window ring slots per sequence
constexpr int kWinSplits = kWinSlots / kT;  // window tiles = extra split workgroups

// One attention problem of a launch: a layer's KV pool, its query, the
// selected positions and where the result goes (the batch view is shared).
struct AttnJob {
  KvLayerDev L;
  const uint16_t *q;         // [B][H][512 + rope]
  const int32_t *idx;        // [B][K]
  uint8_t *win_codes;        // [B][128][512] E4M3 window entries, or null
  float *win_scales;         // [B][128] per-token scales
  const float *win_latent;   // [B][512] the current token's window entry to append first, or null
  float *out;                // [B][H][512]
  float *lse;                // [B][H] or null
};

struct AttnArgs {
  AttnJob job[kMaxAttnJobs];
  SeqsDev S;
  int heads;              // H
  int top_k;
  int splits;             // workgroups per (job, b, head group) along the selected entries
  int parts;              // partials per (job, b, head): splits, plus kWinSplits with the window
  int tiles_per_split;
  float scale_log2;       // softmax scale * log2(e)
  float *part_o;          // [jobs][B][H][parts][512]  (parts > 1)
  float *part_ml;         // [jobs][B][H][parts][2]
  uint32_t *dbg;          // debug flag word, or null
};

// LDS of one workgroup.  LD is the tile row (f16): 512 latent channels (+ 64
// rope) + 8 of padding, so a row is an odd number of 16-byte units (65 or 73)
// and the 16 lanes of a 16-byte access that differ in their entry fall on 16
// different bank groups.
template <int MT, int LD>
struct __attribute__((aligned(16))) Smem {  // 16-byte aligned rows: every tile access is a 128-bit LDS op
  __attribute__((aligned(16))) f16 cq[3][kT][LD];   // row-major dequantized tiles (+ rope), used in turn
  float s[kKParts<MT>][16 * MT][kT + 1];             // partial logits of the k-parts (padded rows)
  // P (hi + lo parts) and the accumulator factors of two tiles: a tile's
  // softmax writes one while the previous tile's PV reads the other
  __attribute__((aligned(16))) f16 p_hi[2][16 * MT][kPLd];
  __attribute__((aligned(16))) f16 p_lo[2][16 * MT][kPLd];
  float alpha[2][16 * MT];
  float m_run[16 * MT], l_run[16 * MT];
  uint32_t slot[kSlotCap];       // physical rows of this workgroup's entries (kNoSlot: skipped)
  float wts[kT], wp[kT];         // window tile: token scales, and times the P normalization
  float unnorm;                  // window tile: the P normalization, inverted
  float wamax[kWaves];           // appended window entry: per-wave amax
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
template <int LD>
__device__ __forceinline__ f16x8 pv_operand(const f16 *p) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * LD));
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

// Raw row fragment of one entry held by one thread: 32 channels of FP4 codes
// (16 bytes), their 2 E4M3 scales and (with rope) 4 rope values.
struct Raw {
  uint4 c;
  uint2 rp;
  uint32_t sc2;
  bool valid;
};

template <int MT, bool ROPE>
__global__ void __launch_bounds__(kThreads) sparse_attn_kernel(AttnArgs a) {
  constexpr int HG = 16 * MT;                  // heads in this workgroup
  constexpr int QW = kLatent + (ROPE ? 64 : 0);  // q row width
  constexpr int LD = ROPE ? kLatent + 64 + 8 : kLatent + 8;  // tile row (f16)
  constexpr int KS = QW / 32;                  // 16 or 18 k-steps of 32 channels
  constexpr int KP = kKParts<MT>;              // waves splitting the k-steps of one logit tile
  constexpr int QKS = (KS + KP - 1) / KP;      // k-steps per wave (the last part may be shorter)
  // M-tiles (16 heads) x N-tiles (16 entries) of one wave's QK^T: with 64
  // heads and no rope a wave takes 2 M-tiles of one N-tile, so each K
  // fragment it reads from LDS feeds two MFMAs (the tile is read twice per
  // pass, not 4x); with rope the second M-tile's q fragments would not fit in
  // registers, so a wave takes one M-tile of both N-tiles
  constexpr int QMT = MT == 4 && !ROPE ? 2 : 1;
  constexpr int QNT = MT == 4 && ROPE ? 2 : 1;
  constexpr bool kEvenParts = KS % KP == 0;    // every k-part has QKS k-steps
  __shared__ Smem<MT, LD> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, hg = blockIdx.y;
  const int jz = blockIdx.z, jn = jz / a.S.batch, b = jz - jn * a.S.batch;  // job, sequence
  const AttnJob &J = a.job[jn];
  const int h0 = hg * HG;
  const size_t hrow0 = (size_t)jz * a.heads + h0;  // first (job, b, head) row of this workgroup
  const int n = min(max(a.S.seq_lens[b], 0), a.S.max_len);
  // workgroups past the selection's splits take window tile split - splits:
  // ring slots 32 wt .. 32 wt + 31, valid below min(seq_len, 128)
  const bool win = split >= a.splits;
  const int wt = split - a.splits;
  const int nwin = min(max(a.S.seq_lens[b], 0), kWinSlots);
  const int s_new = nwin > 0 ? (a.S.seq_lens[b] - 1) % kWinSlots : -1;  // the current token's slot
  const bool pack_new = win && J.win_latent != nullptr && s_new >= 0 && s_new / kT == wt;

  const int n_tiles_all = (a.top_k + kT - 1) / kT;
  const int tile_begin = win ? 0 : split * a.tiles_per_split;
  const int tile_end = win ? (nwin > kT * wt ? 1 : 0) : min(tile_begin + a.tiles_per_split, n_tiles_all);
  const int e_begin = tile_begin * kT;
  // <= kSlotCap (host-chosen splits)
  const int e_count = win ? kT : max(0, min(tile_end * kT, a.top_k) - e_begin);
  const int32_t *idx_row = J.idx + (size_t)b * a.top_k;

  // ---- QK^T work of this wave: M-tiles qk_mt .. qk_mt + QMT - 1 (16 heads
  // each), N-tiles qk_nt0 .. qk_nt0 + QNT - 1 (16 entries each), k-part qk_kp
  // (k-steps qk_k0 .. qk_k1 - 1);
  // the KP partial logits of an entry are added when the softmax reads them
  int qk_mt, qk_nt0, qk_kp;
  if constexpr (MT == 4 && QMT == 2) { qk_mt = 2 * (wave & 1); qk_nt0 = (wave >> 1) & 1; qk_kp = wave >> 2; }
  else if constexpr (MT == 4) { qk_mt = wave & 3; qk_nt0 = 0; qk_kp = wave >> 2; }
  else if constexpr (MT == 2) { qk_mt = wave & 1; qk_nt0 = (wave >> 1) & 1; qk_kp = wave >> 2; }
  else { qk_mt = 0; qk_nt0 = wave & 1; qk_kp = wave >> 1; }
  const int qk_k0 = qk_kp * QKS;
  const int qk_kn = min(QKS, KS - qk_k0);  // k-steps of this part (uniform)

  // ---- entry indices of this workgroup, then their physical rows (two dependent
  // reads for all entries at once; the q loads below overlap them)
  constexpr int kRounds = kSlotCap / kThreads;
  int pos[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) pos[j] = -1;
  if (!win) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (kThreads * j >= e_count) break;  // uniform: rounds past this workgroup's entries are not read
      const int i = kThreads * j + tid;
      const int p = idx_row[min(e_begin + i, a.top_k - 1)];  // clamped read, masked below
      pos[j] = i < e_count ? p : -1;
      if (a.dbg != nullptr && i < e_count && (p < -1 || p >= n)) dbg_raise(a.dbg, kDbgIndex);
    }
  }

  // q fragments (A operand) of M-tile qk_mt + i: head 16*(qk_mt + i) + lane%16,
  // channels 32*(qk_k0 + ks) + 8*(lane/16) .. +7
  f16x8 qf[QMT][QKS];
  {
    uint4 raw[QMT][QKS];
#pragma unroll
    for (int i = 0; i < QMT; ++i) {
      const uint16_t *qrow =
          J.q + ((size_t)b * a.heads + h0 + 16 * (qk_mt + i) + (lane & 15)) * QW + 32 * qk_k0 + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks)
        raw[i][ks] = (kEvenParts || ks < qk_kn) ? *reinterpret_cast<const uint4 *>(qrow + 32 * ks)
                                                : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < QMT; ++i)
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks) qf[i][ks] = bf16x8_to_f16x8(raw[i][ks]);
    if (a.dbg != nullptr) {  // a bf16 magnitude above fp16's largest finite value (65504)
      bool big = false;
#pragma unroll
      for (int i = 0; i < QMT; ++i)
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) big |= !(fabsf((float)qf[i][ks][e]) <= 65504.0f);
      if (big) dbg_raise(a.dbg, kDbgQRange);
      if (split == 0 && hg == 0 && tid == 0 && (J.L.num_blocks < 0 || a.S.seq_lens[b] < 0 ||
                                                  a.S.seq_lens[b] > a.S.max_len))
        dbg_raise(a.dbg, kDbgSeqLen);
    }
  }

  if (!win) {
    int blk[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (kThreads * j >= e_count) break;  // (slots past e_count are never read)
      const int p = pos[j];
      const bool ok = p >= 0 && p < n && p / kPage < a.S.max_blocks;
      // clamped read, masked below (a table without columns maps nothing)
      blk[j] = a.S.max_blocks > 0 ? a.S.block_table[(size_t)b * a.S.max_blocks + (ok ? p / kPage : 0)] : -1;
      pos[j] = ok ? p : -1;
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (kThreads * j >= e_count) break;
      const int i = kThreads * j + tid;
      const bool ok = pos[j] >= 0 && blk[j] >= 0 && blk[j] < J.L.num_blocks;
      if (a.dbg != nullptr && pos[j] >= 0 && !ok) dbg_raise(a.dbg, kDbgPage);
      sm.slot[i] = ok ? (uint32_t)blk[j] * kPage + (uint32_t)(pos[j] % kPage) : kNoSlot;
    }
  } else {
    // appending the current token's entry (slot (n - 1) mod 128) when this tile holds it: FP8 pack with
    // s = amax / 448, code = E4M3(x / s); thread t packs channel t
    float snew = 0.0f;
    if (pack_new) {
      const float x = J.win_latent[(size_t)b * kLatent + tid];
      float m = fabsf(x);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) sm.wamax[wave] = m;
      __syncthreads();  // uniform: the whole workgroup packs
      float amax = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, sm.wamax[w]);
      snew = __fdiv_rn(amax, 448.0f);
      uint32_t c = 0u;
      if (snew > 0.0f) c = e4m3_encode(fabsf(__fdiv_rn(x, snew))) | ((__float_as_uint(x) >> 31) << 7);
      sm.newc[tid] = (uint8_t)c;
      if (hg == 0) {  // one head group writes the ring
        J.win_codes[((size_t)b * kWinSlots + s_new) * kLatent + tid] = (uint8_t)c;
        if (tid == 0) J.win_scales[(size_t)b * kWinSlots + s_new] = snew;
      }
    }
    if (tid < kT) {
      // window tile: ring slots, token scales, and a power of two that brings the
      // tile's largest token scale into [1, 2) (P times the scale stays in fp16's
      // normal range)
      const int s = kT * wt + tid;
      const bool ok = s < nwin;
      sm.slot[tid] = ok ? (uint32_t)s : kNoSlot;
      const float ts = !ok ? 0.0f : (pack_new && s == s_new) ? snew : J.win_scales[(size_t)b * kWinSlots + s];
      float mx = ts;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
      const float norm = mx > 0.0f ? __uint_as_float((254u - ((__float_as_uint(mx) >> 23) & 0xFFu)) << 23) : 1.0f;
      sm.wts[tid] = ts;
      sm.wp[tid] = ts * norm;
      if (tid == 0) sm.unnorm = 1.0f / norm;
    }
  }

  // ---- PV accumulators: wave owns channels [64*wave, 64*wave+64) for all HG heads
  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // slot[] is complete

  // gather of one tile: thread -> entry tile_entry, channels 32 tile_chunk ..
  // + 31 (16 bytes of codes, 2 scales, 4 rope values).  Within a wave the 16
  // lanes of one chunk hold 16 different entries, so each 16-byte LDS store of
  // the dequantized tile (rows of an odd number of 16-byte units) hits 16
  // different bank groups; the 4 lanes l, l + 16, l + 32, l + 48 read 64
  // contiguous bytes of one row.  Every load is issued unconditionally (a
  // skipped entry reads row 0 and is zeroed when dequantized; an empty pool
  // never launches a tile).
  const int tile_entry = (lane & 15) + 16 * (wave & 1), tile_chunk = (lane >> 4) + 4 * (wave >> 1);
  auto load_raw = [&](int tile, Raw &r) {
    const int li = tile * kT + tile_entry - e_begin;
    const uint32_t slot = li < e_count ? sm.slot[li] : kNoSlot;
    const size_t rs = slot == kNoSlot ? 0 : slot;
    r.c = *reinterpret_cast<const uint4 *>(J.L.codes + rs * (kLatent / 2) + 16 * tile_chunk);
    r.sc2 = *reinterpret_cast<const uint16_t *>(J.L.scales + rs * (kLatent / kGroup) + 2 * tile_chunk);
    if constexpr (ROPE) r.rp = *reinterpret_cast<const uint2 *>(J.L.rope + rs * 64 + 4 * tile_chunk);
    r.valid = slot != kNoSlot;
  };

  // dequantize one tile's row fragments into a row-major tile buffer
  // (branch-free: a skipped entry is masked to scale 0 and rope 0, so its
  // channels are all zero; the two E4M3 scales go through the hardware fp8
  // convert, exact in fp16)
  auto dequant = [&](const Raw &r, f16 (*cq)[LD]) {
    const uint32_t vmask = 0u - (uint32_t)r.valid;
    const uint32_t words[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
    const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sc2 & vmask, 1.0f, false);  // scale bytes 0, 1
#pragma unroll
    for (int wi = 0; wi < 4; ++wi)
      *reinterpret_cast<f16x8 *>(&cq[tile_entry][32 * tile_chunk + 8 * wi]) = deq8(words[wi], s01[wi >> 1]);
    if constexpr (ROPE) {
      const uint2 rp = make_uint2(r.rp.x & vmask, r.rp.y & vmask);
      f16 rh[4];
      rh[0] = (f16)__uint_as_float(rp.x << 16);
      rh[1] = (f16)__uint_as_float(rp.x & 0xFFFF0000u);
      rh[2] = (f16)__uint_as_float(rp.y << 16);
      rh[3] = (f16)__uint_as_float(rp.y & 0xFFFF0000u);
      typedef f16 f16x4 __attribute__((ext_vector_type(4)));
      *reinterpret_cast<f16x4 *>(&cq[tile_entry][kLatent + 4 * tile_chunk]) = f16x4{rh[0], rh[1], rh[2], rh[3]};
      if (a.dbg != nullptr) {
        bool big = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) big |= !(fabsf((float)rh[i]) <= 65504.0f);
        if (big) dbg_raise(a.dbg, kDbgQRange);
      }
    }
  };

  // online-softmax state: thread -> head tid / TPH, entries (tid % TPH) * EPT ..
  // + EPT - 1 of a tile; the TPH threads of a head keep the same running max
  // and sum in registers (threads past HG * TPH take no part)
  constexpr int TPH = (kThreads / HG) < 16 ? (kThreads / HG) : 16;  // threads per head (8 or 16)
  constexpr int EPT = kT / TPH;   // entries per thread (4 or 2)
  const int sm_h = tid / TPH, sm_part = tid % TPH;
  const bool sm_on = tid < HG * TPH;
  float m_run = -INFINITY, l_run = 0.f;

  // O = alpha * O + P V for a tile whose softmax is done: tile buffer cq, P
  // and alpha buffer pb (wave: channels 64*wave .. +63, all heads)
  auto pv = [&](f16 (*cq)[LD], int pb) {
    float al[MT][4];
    bool rescale = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        al[mt][rr] = sm.alpha[pb][16 * mt + 4 * (lane >> 4) + rr];
        rescale |= al[mt][rr] != 1.f;
      }
    if (__ballot(rescale)) {  // 16 * MT multiplies per lane: skipped unless some row's reference moved
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[mt][nt][rr] *= al[mt][rr];
    }
    f16x8 ph[MT], pl[MT], bv[4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ph[mt] = lds_f16x8(&sm.p_hi[pb][16 * mt + (lane & 15)][8 * (lane >> 4)]);
      pl[mt] = lds_f16x8(&sm.p_lo[pb][16 * mt + (lane & 15)][8 * (lane >> 4)]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bv[nt] = pv_operand<LD>(&cq[8 * (lane >> 4) + ((lane >> 2) & 3)][64 * wave + 16 * nt + 4 * (lane & 3)]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[mt], bv[nt], acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[mt], bv[nt], acc[mt][nt], 0, 0, 0);
      }
  };

  // online softmax of one tile: logit = scale * (sum of the k-parts), masked
  // entries -inf; writes P and alpha buffer pb
  auto softmax = [&](int tile, int pb) {
    if (sm_on) {
      float v[EPT];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int ent = sm_part * EPT + i;
        float x = sm.s[0][sm_h][ent];
#pragma unroll
        for (int kp = 1; kp < KP; ++kp) x += sm.s[kp][sm_h][ent];
        const int li = tile * kT + ent - e_begin;
        const bool valid = li < e_count && sm.slot[li] != kNoSlot;
        float es = a.scale_log2;
        if (win) es *= sm.wts[ent];  // window entries: the token scale of the E4M3 codes
        v[i] = valid ? x * es : -INFINITY;
        mx = fmaxf(mx, v[i]);
      }
      mx = group_max<TPH>(mx);
      // The reference m_run moves only when a logit exceeds it by more than
      // 2^8 (in the exp2 domain): weights stay below 2^8, O and l are left
      // unscaled on most tiles, and O / l is the same ratio.
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      float sum = 0.f;
      typedef f16 f16xE __attribute__((ext_vector_type(EPT)));
      f16xE ph, pl;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const float pv = (m_new == -INFINITY) ? 0.f : exp2f(v[i] - m_new);
        sum += pv;
        // window: P times the token scale.  pw is rounded to fp32 once and
        // both parts are split from that value: left visible, the product
        // gets folded into one fp16 conversion (rounded once from the exact
        // product) but not the other, and hi + lo can miss pw by one fp16 ulp
        float pw = win ? pv * sm.wp[sm_part * EPT + i] : pv;
        asm volatile("" : "+v"(pw));
        ph[i] = (f16)pw;
        pl[i] = (f16)(pw - (float)ph[i]);
      }
      *reinterpret_cast<f16xE *>(&sm.p_hi[pb][sm_h][sm_part * EPT]) = ph;
      *reinterpret_cast<f16xE *>(&sm.p_lo[pb][sm_h][sm_part * EPT]) = pl;
      sum = group_sum<TPH>(sum);
      // (from an empty state O and l are zero: no rescaling either)
      const float al = (m_new == m_run || m_run == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      l_run = l_run * al + sum;
      m_run = m_new;
      if (sm_part == 0) sm.alpha[pb][sm_h] = al;
    }
  };

  // One tile from buffer cq in two phases, each ended by a barrier:
  //   1. its partial logits (QK^T, matrix cores) and the next tile's
  //      dequantization into cq_next (vector ALU);
  //   2. the previous tile's PV from cq_prev (matrix cores) beside this
  //      tile's online softmax (vector ALU), which writes the other P buffer.
  // The last tile's PV follows the loop.  Three tile buffers in turn: the one
  // a phase writes was last read two barriers earlier.
  auto step = [&](int tile, f16 (*cq)[LD], bool has_next, const Raw &next, f16 (*cq_next)[LD],
                  f16 (*cq_prev)[LD]) {
    const int pb = (tile - tile_begin) & 1;  // this tile's P buffer
    auto qk = [&]() {
      // 1. partial logits S_kp = Q C^T over this wave's k-part; even and odd
      // k-steps of every N-tile accumulate separately (2 or 4 independent MFMA
      // chains), the B fragments of 4 k-steps read together ahead of them
      f32x4 sacc[QMT][QNT][2];
      const f16 *brow[QNT];
#pragma unroll
      for (int j = 0; j < QNT; ++j) {
#pragma unroll
        for (int i = 0; i < QMT; ++i) {
          sacc[i][j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
          sacc[i][j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        brow[j] = &cq[16 * (qk_nt0 + j) + (lane & 15)][32 * qk_k0 + 8 * (lane >> 4)];
      }
#pragma unroll
      for (int k0 = 0; k0 < QKS; k0 += 4) {
        f16x8 bq[QNT][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < QNT; ++j)
            if (k0 + kk < QKS)
              bq[j][kk] = (kEvenParts || k0 + kk < qk_kn) ? lds_f16x8(brow[j] + 32 * (k0 + kk)) : f16x8{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < QNT; ++j)
#pragma unroll
            for (int i = 0; i < QMT; ++i)
              if (k0 + kk < QKS)
                sacc[i][j][kk & 1] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[i][k0 + kk], bq[j][kk], sacc[i][j][kk & 1], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < QNT; ++j)
#pragma unroll
        for (int i = 0; i < QMT; ++i) {
          const int nt = qk_nt0 + j;
          const f32x4 sa = sacc[i][j][0] + sacc[i][j][1];
          // lane holds S_kp[head 16*mt + 4*(lane/16) + r][entry 16*nt + lane%16]
          const int ent = 16 * nt + (lane & 15);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sm.s[qk_kp][16 * (qk_mt + i) + 4 * (lane >> 4) + rr][ent] = sa[rr];
        }
    };
    qk();
    if (has_next) dequant(next, cq_next);
    __syncthreads();
    if (tile > tile_begin) pv(cq_prev, pb ^ 1);
    softmax(tile, pb);
    __syncthreads();
  };

  // ---- tiles: three register sets of raw rows (each tile's loads are issued
  // three tiles ahead; loads past the last tile re-read the last tile) and
  // three tile buffers, so the unrolled loop keeps both in step
  if (win) {
    if (tile_begin < tile_end) {
      // the window tile: thread -> entry tile_entry, channels 32 tile_chunk .. + 31
      // (32 E4M3 bytes), converted to fp16 (exact); skipped slots and the rope
      // part are zero
      const uint32_t slot = sm.slot[tile_entry];
      const uint4 *cp = pack_new && slot == (uint32_t)s_new  // the appended entry, from LDS
                            ? reinterpret_cast<const uint4 *>(sm.newc + 32 * tile_chunk)
                            : reinterpret_cast<const uint4 *>(J.win_codes +
                                                              ((size_t)b * kWinSlots + (slot == kNoSlot ? 0 : slot)) *
                                                                  kLatent +
                                                              32 * tile_chunk);
      uint4 w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) w[i] = cp[i];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f16x8 lo = fp8x8_to_f16(make_uint2(w[i].x, w[i].y));
        f16x8 hi = fp8x8_to_f16(make_uint2(w[i].z, w[i].w));
        if (slot == kNoSlot) lo = hi = f16x8{};
        *reinterpret_cast<f16x8 *>(&sm.cq[0][tile_entry][32 * tile_chunk + 16 * i]) = lo;
        *reinterpret_cast<f16x8 *>(&sm.cq[0][tile_entry][32 * tile_chunk + 16 * i + 8]) = hi;
      }
      if constexpr (ROPE) {
        typedef f16 f16x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<f16x4 *>(&sm.cq[0][tile_entry][kLatent + 4 * tile_chunk]) = f16x4{};
      }
      __syncthreads();
      step(0, sm.cq[0], false, Raw{}, sm.cq[1], sm.cq[2]);
      pv(sm.cq[0], 0);
    }
  } else if (tile_begin < tile_end && J.L.num_blocks > 0) {
    const int last = tile_end - 1;
    Raw ra, rb, rc;
    load_raw(tile_begin, ra);
    load_raw(min(tile_begin + 1, last), rb);
    load_raw(min(tile_begin + 2, last), rc);
    dequant(ra, sm.cq[0]);
    load_raw(min(tile_begin + 3, last), ra);
    __syncthreads();
    for (int tile = tile_begin; tile < tile_end; tile += 3) {
      step(tile, sm.cq[0], tile + 1 < tile_end, rb, sm.cq[1], sm.cq[2]);
      load_raw(min(tile + 4, last), rb);
      if (tile + 1 < tile_end) {
        step(tile + 1, sm.cq[1], tile + 2 < tile_end, rc, sm.cq[2], sm.cq[0]);
        load_raw(min(tile + 5, last), rc);
      }
      if (tile + 2 < tile_end) {
        step(tile + 2, sm.cq[2], tile + 3 < tile_end, ra, sm.cq[0], sm.cq[1]);
        load_raw(min(tile + 6, last), ra);
      }
    }
    pv(sm.cq[(last - tile_begin) % 3], (last - tile_begin) & 1);  // the last tile's PV
  }
  if (sm_on && sm_part == 0) {
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
      const size_t h = hrow0 + hl;  // partial row (job, b, head)
      float sc = win ? sm.unnorm : 1.0f;
      float *dst = a.part_o + (h * a.parts + split) * kLatent;
      if (final_out) {
        const float l = sm.l_run[hl];
        sc = l > 0.f ? 1.0f / l : 0.f;
        dst = J.out + ((size_t)b * a.heads + h0 + hl) * kLatent;
      }
      dst += 64 * wave + (lane & 15);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dst[16 * nt] = acc[mt][nt][r] * sc;
    }
  if (final_out) {
    if (J.lse != nullptr && tid < HG) {
      const float l = sm.l_run[tid];
      J.lse[(size_t)b * a.heads + h0 + tid] = l > 0.f ? (sm.m_run[tid] + log2f(l)) / kLog2e : -INFINITY;
    }
  } else if (tid < HG) {
    float *ml = a.part_ml + ((hrow0 + tid) * a.parts + split) * 2;
    ml[0] = sm.m_run[tid];
    ml[1] = sm.l_run[tid];
  }
}

// Merges the splits' partials: workgroup (b*H + h, half) of one full wave
// covers 256 channels of one head, one float4 per thread.  Splits are read 8
// at a time (all loads of a chunk issued together) and merged online.
constexpr int kCombineThreads = 64;
// Where the merged rows go: partial row r = (job, b, head) belongs to job
// r / rows_per_job and is row r % rows_per_job of that job's out / lse.
struct CombineOut {
  float *out[kMaxAttnJobs];
  float *lse[kMaxAttnJobs];
  int rows_per_job;  // B * H
};

__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int splits,
                                                          CombineOut co) {
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
  const int jn = bh / co.rows_per_job, row = bh - jn * co.rows_per_job;
  reinterpret_cast<float4 *>(co.out[jn] + (size_t)row * kLatent)[c4] =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  float *lse = co.lse[jn];
  if (lse != nullptr && quarter == 0 && tid == 0) lse[row] = l > 0.f ? (m + log2f(l)) / kLog2e : -INFINITY;
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
                                                          CombineOut co) {
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
    const int jn = bh / co.rows_per_job, row = bh - jn * co.rows_per_job;
    reinterpret_cast<float4 *>(co.out[jn] + (size_t)row * kLatent)[kWideCols * q + tid] =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    float *lse = co.lse[jn];
    if (lse != nullptr && q == 0 && tid == 0) lse[row] = lt > 0.f ? (mx + log2f(lt)) / kLog2e : -INFINITY;
  }
}

// Heads per workgroup.  64 shares each dequantized tile (and each window
// tile) among the most heads; fewer heads per workgroup give more
// workgroups, each with less MFMA work per tile (the tile is then
// dequantized once per head group, from L2).  Measured per step (64 heads
// per problem): one sequence over 4 layers 72 us with 16, 74 with 32, 78
// with 64; 8 sequences of one layer 55 us with 32, 57 with 64, 62 with 16
// (the 32-head groups take half as many splits, so the combine reads half
// the partials); one sequence over 20 layers the same with 32 or 64, and 64
// won over 16 with their windows (99 -> 93 us).
// `problems` counts (job, sequence) pairs of the launch.
int heads_per_group(int problems, int heads) {
  if (heads % 64 == 0) {
    const int64_t groups64 = (int64_t)problems * (heads / 64);
    if (groups64 >= 16) return 64;
    if (groups64 >= 8) return 32;
  }
  return 16;
}

// Bytes of the split partials (out, then m and l) of a launch.
size_t partial_bytes(int problems, int heads, int parts) {
  if (parts == 1) return 256;
  const size_t rows = (size_t)problems * heads * parts;
  const size_t o = rows * kLatent * sizeof(float);
  const size_t ml = rows * 2 * sizeof(float);
  return ((o + 255) & ~(size_t)255) + ((ml + 255) & ~(size_t)255);
}

// Split-K workgroups per (problem, head group); with a bound on the partials'
// bytes (the allocation-free entry point's scratch) the count is lowered
// until they fit, down to the least a workgroup's slot array allows.
int choose_splits(int problems, int heads, int top_k, bool window, size_t max_bytes) {
  const int hpg = heads_per_group(problems, heads);
  const int groups = problems * (heads / hpg);
  const int tiles = (top_k + kT - 1) / kT;
  int splits = (256 + groups - 1) / groups;  // about one workgroup per CU
  // a 64-head workgroup's slot resolution and first gather cost as much as a
  // tile or two: give each at least two tiles
  if (hpg == 64 && splits > (tiles + 1) / 2) splits = (tiles + 1) / 2;
  if (splits > tiles) splits = tiles;
  if (splits > kMaxSplits) splits = kMaxSplits;
  const int min_splits = (tiles * kT + kSlotCap - 1) / kSlotCap;  // a workgroup resolves at most kSlotCap entries
  if (splits < min_splits) splits = min_splits;
  if (splits < 1) splits = 1;
  const int win = window ? kWinSplits : 0;
  while (splits > min_splits && splits > 1 && partial_bytes(problems, heads, splits + win) > max_bytes) --splits;
  return splits;
}

}  // namespace

size_t attn_workspace_bytes(int jobs, int batch, int heads, int top_k, bool window, size_t max_bytes) {
  const int problems = jobs * batch;
  const int parts = choose_splits(problems, heads, top_k, window, max_bytes) + (window ? kWinSplits : 0);
  return partial_bytes(problems, heads, parts);
}

hipError_t launch_sparse_attn(const AttnLaunchJob *jobs, int n_jobs, const SeqsDev &S, int heads, int top_k,
                              float scale, void *ws, size_t max_ws, hipStream_t st) {
  if (S.batch == 0 || n_jobs == 0) return hipSuccess;
  const bool window = jobs[0].win_codes != nullptr;
  const int problems = n_jobs * S.batch;
  const int hgsz = heads_per_group(problems, heads);
  const int splits = choose_splits(problems, heads, top_k, window, max_ws);
  const int parts = splits + (window ? kWinSplits : 0);
  const int tiles = (top_k + kT - 1) / kT;
  AttnArgs a;
  for (int j = 0; j < n_jobs; ++j) {
    const AttnLaunchJob &x = jobs[j];
    a.job[j] = AttnJob{x.L, x.q, x.indices, x.win_codes, x.win_scales, x.win_latent, x.out, x.lse};
  }
  a.S = S;
  a.heads = heads;
  a.top_k = top_k;
  a.splits = splits;
  a.parts = parts;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  a.scale_log2 = scale * kLog2e;
  a.dbg = debug_flags();
  const size_t rows = (size_t)problems * heads * parts;
  const size_t o_bytes = rows * kLatent * sizeof(float);
  a.part_o = static_cast<float *>(ws);
  a.part_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + ((o_bytes + 255) & ~(size_t)255));
  const dim3 grid(parts, heads / hgsz, problems);
  timer_before(kKernSparseAttn, st);
  const bool rope = jobs[0].L.rope_dim != 0;
  if (hgsz == 64) {
    if (rope) sparse_attn_kernel<4, true><<<grid, dim3(kThreads), 0, st>>>(a);
    else sparse_attn_kernel<4, false><<<grid, dim3(kThreads), 0, st>>>(a);
  } else if (hgsz == 32) {
    if (rope) sparse_attn_kernel<2, true><<<grid, dim3(kThreads), 0, st>>>(a);
    else sparse_attn_kernel<2, false><<<grid, dim3(kThreads), 0, st>>>(a);
  } else {
    if (rope) sparse_attn_kernel<1, true><<<grid, dim3(kThreads), 0, st>>>(a);
    else sparse_attn_kernel<1, false><<<grid, dim3(kThreads), 0, st>>>(a);
  }
  timer_after(kKernSparseAttn, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts == 1) return e;
  CombineOut co;
  for (int j = 0; j < n_jobs; ++j) {
    co.out[j] = jobs[j].out;
    co.lse[j] = jobs[j].lse;
  }
  co.rows_per_job = S.batch * heads;
  const int prow = problems * heads;
  timer_before(kKernAttnCombine, st);
  const dim3 wide_grid(prow, kLatent / 4 / kWideCols);
  if (parts > 32)
    attn_combine_wide_kernel<3><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, co);
  else if (parts > 16)
    attn_combine_wide_kernel<2><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, co);
  else if (parts > 8)
    attn_combine_wide_kernel<1><<<wide_grid, dim3(kWideThreads), 0, st>>>(a.part_o, a.part_ml, parts, co);
  else
    attn_combine_kernel<<<dim3(prow, kLatent / 4 / kCombineThreads), dim3(kCombineThreads), 0, st>>>(
        a.part_o, a.part_ml, parts, co);
  timer_after(kKernAttnCombine, st);
  return hipGetLastError();
}

}  // namespace csa2
