// Indexer scoring, exact top-K selection and the hierarchical candidate pool.
//
// Sources: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "CSA2"
// (Full / Reindex / Reuse modes: Full and Reindex score cached indexer keys
// with their own query and select the top-K; Reuse selects nothing) and
// section "Hierarchical Sparse Indexer" (the first Full layer scores every
// visible position, selects its own top-K and, in the same pass, gives each
// block of 8 positions the maximum score inside it and keeps the best 2048
// blocks -- at most 16,384 positions -- as the candidate pool that the later
// Reindex layers score).
//
// Design (ours; the pages give no kernel).  A score is an fp32 dot product
// (fp32 or bf16 keys, fp32 query) mapped to an order-preserving 32-bit key;
// item order is (key descending, position ascending), so ties go to the lower
// position.  No global atomics, fences or inter-workgroup waits are used: on
// gfx950 they cost more than a kernel boundary.
//   producers  Each workgroup owns a fixed slice of a row (2048 or 1024
//              positions of a full scan, 2048 given scores, or 16 pool blocks),
//              keeps its keys in LDS and stores all of them.  It then emits its
//              best items as a candidate segment, cut exactly to a budget of
//              about 3x its expected share of the top-K, plus the segment's
//              edge: every item it did not emit has a key below the edge.  The
//              cut uses one histogram level of bins counted down from the
//              slice's largest key (2^12 key units wide, 2^14 for the
//              multi-head FP4 scores) when the budget is small (the common
//              decode case), else two 11-bit radix levels of the absolute key.
//              The full scan streams the keys with non-temporal 16-byte loads,
//              16 in flight per lane, after one page-table lookup per 64
//              positions; loads are never guarded by branches (unmapped pages
//              read slot 0 and are masked).  In hierarchical mode it emits two
//              segments: block maxima and positions.
//   select     One 512-thread workgroup per row and output loads the segments
//              into registers in position order and finds the exact threshold
//              with a 2048-bin histogram over the candidates' own key range,
//              a second one inside the boundary bin and an exact rank of the
//              few items left, or one LDS maximum when one of them is taken
//              (radix levels on key then position bits when heavy ties leave
//              more; each threshold search runs in one wave).  A segment
//              whose edge exceeds the threshold's key may
//              hold more winners: those segments are re-read in full from the
//              stored keys (items at or above the threshold key only) and the
//              threshold is recomputed, which is then exact.  If that would
//              not fit in LDS, the select runs over every stored item of the
//              row.  Outputs are written in increasing position order and
//              padded with -1, so results are deterministic.
//   Hierarchical Full: the block select (pool) and the position select (the
//   layer's own top-K over all positions) run as two workgroups side by side.
//   Reindex: 16-block producer workgroups score the pool with the layer's own
//   query; the select runs as above.
#include "append.h"
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int kBins = 2048;                    // 11-bit radix digits
constexpr int kScanPos = 2048;                 // positions per producer workgroup (1024 for small grids)
constexpr int kScanPages = kScanPos / kPage;   // 32
constexpr int kBlk = 8;                        // positions per pool block
constexpr int kScanBlocks = kScanPos / kBlk;   // 256
constexpr int kCandCap = 6144;                 // candidates one select workgroup holds in LDS
constexpr int kSelThreads = 512;
constexpr int kSelIPT = kCandCap / kSelThreads;  // 12
constexpr int kPoolBlocksPerWg = 16;           // pool producer: 16 blocks = 128 items
constexpr int kPoolItemsPerWg = kPoolBlocksPerWg * kBlk;
constexpr int kMaxPoolItems = 2048 * kBlk;     // 16,384
constexpr int kMaxSeg = 4096;                  // segments per row (8M positions, host-validated)
constexpr int kSegPerThread = kMaxSeg / kSelThreads;  // 8
constexpr int kMaxIdxJobs = kMaxIdxLayers;     // Reindex layers scored by one launch

enum SelMode { kFullPos = 0, kFullHier = 1, kReindex = 2, kGiven = 3 };

struct SegInfo {
  uint32_t count;  // candidates emitted
  uint32_t edge;   // every item the segment did not emit has a key < edge
};

// Per-row workspace views.
struct SelWs {
  uint32_t *keys;    // [B][cap_keys]      position keys (scan) or keys of given scores
  uint32_t *bkeys;   // [B][cap_blocks]    block-max keys (hierarchical scan)
  uint2 *pool_full;  // [B][kMaxPoolItems] (key, position) of every pool item (Reindex)
  uint2 *cand_pos;   // [B][kCandCap]      position candidates
  uint2 *cand_blk;   // [B][kCandCap]      block candidates
  SegInfo *seg_pos;  // [B][max_seg]
  SegInfo *seg_blk;  // [B][max_seg]
  int64_t cap_keys, cap_blocks;
  int max_seg;
  int slice;         // positions per producer segment (scan: 1024 or 2048; given scores: 2048)
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct WsShape {
  int64_t cap_keys, cap_blocks;
  int max_seg;
  int slice;
  bool pool;
};

// Producer segments of a full scan are 2048 positions, or 1024 when 2048
// would leave at most one scan workgroup per CU (256): two workgroups per CU
// then overlap one's emission with the other's key loads.  Given scores
// always use 2048.
WsShape ws_shape(int batch, int max_len, int pool_blocks, bool scan) {
  WsShape s;
  s.cap_keys = round_up(max_len > 0 ? max_len : 1, kScanPos);
  s.cap_blocks = round_up((s.cap_keys + kBlk - 1) / kBlk, kScanBlocks);
  s.slice = (scan && (int64_t)(batch > 0 ? batch : 1) * (s.cap_keys / kScanPos) <= 256) ? kScanPos / 2 : kScanPos;
  const int seg_scan = (int)(s.cap_keys / s.slice);
  const int seg_pool = (pool_blocks + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg;
  s.max_seg = seg_scan > seg_pool ? seg_scan : seg_pool;
  s.pool = pool_blocks > 0;
  return s;
}

size_t ws_bytes_for(int batch, const WsShape &s) {
  const size_t B = (size_t)batch;
  return align256(4 * B * s.cap_keys) + align256(4 * B * s.cap_blocks) +
         (s.pool ? align256(8 * B * kMaxPoolItems) : 0) + 2 * align256(8 * B * kCandCap) +
         2 * align256(sizeof(SegInfo) * B * s.max_seg);
}

SelWs carve(void *ws, int batch, const WsShape &s) {
  const size_t B = (size_t)batch;
  char *p = static_cast<char *>(ws);
  SelWs w;
  w.keys = reinterpret_cast<uint32_t *>(p);
  p += align256(4 * B * s.cap_keys);
  w.bkeys = reinterpret_cast<uint32_t *>(p);
  p += align256(4 * B * s.cap_blocks);
  w.pool_full = nullptr;
  if (s.pool) {
    w.pool_full = reinterpret_cast<uint2 *>(p);
    p += align256(8 * B * kMaxPoolItems);
  }
  w.cand_pos = reinterpret_cast<uint2 *>(p);
  p += align256(8 * B * kCandCap);
  w.cand_blk = reinterpret_cast<uint2 *>(p);
  p += align256(8 * B * kCandCap);
  w.seg_pos = reinterpret_cast<SegInfo *>(p);
  p += align256(sizeof(SegInfo) * B * s.max_seg);
  w.seg_blk = reinterpret_cast<SegInfo *>(p);
  w.cap_keys = s.cap_keys;
  w.cap_blocks = s.cap_blocks;
  w.max_seg = s.max_seg;
  w.slice = s.slice;
  return w;
}

// Workspace of one Reindex layer of a multi-layer call: only the pool items,
// candidates and segment infos (no per-position keys).
constexpr int kPoolSegs = kMaxPoolItems / kPoolItemsPerWg;  // 128
size_t reindex_job_bytes(int batch) {
  const size_t B = (size_t)batch;
  return align256(8 * B * kMaxPoolItems) + align256(8 * B * kCandCap) + align256(sizeof(SegInfo) * B * kPoolSegs);
}

SelWs carve_reindex(void *ws, int batch) {
  const size_t B = (size_t)batch;
  char *p = static_cast<char *>(ws);
  SelWs w{};
  w.pool_full = reinterpret_cast<uint2 *>(p);
  p += align256(8 * B * kMaxPoolItems);
  w.cand_pos = reinterpret_cast<uint2 *>(p);
  p += align256(8 * B * kCandCap);
  w.seg_pos = reinterpret_cast<SegInfo *>(p);
  w.max_seg = kPoolSegs;
  return w;
}

// Candidate budget of a segment: about 3x its expected share of `need`
// winners (at least 8), at most its size and its share of the LDS capacity.
__device__ __forceinline__ int seg_budget(int need, int nseg, int ips) {
  nseg = nseg > 0 ? nseg : 1;
  int c = (3 * need + nseg - 1) / nseg;
  if (c < 8) c = 8;
  if (c > ips) c = ips;
  const int lim = kCandCap / nseg;
  return c < lim ? c : lim;
}

// ------------------------------------------------------------------ scoring
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct KeyLoad {
  u32x4 a, b;  // bf16 keys use a only
};

// Lane l works on position l/8 of an aligned run of 8 and on dims 8*(l%8) ..
// +7 of its key; the 8 partial sums of a position are combined with three DPP
// lane moves, so every lane ends with its position's score.
template <bool F32>
__device__ __forceinline__ KeyLoad load_unit(const void *keys, int64_t slot0, int lane) {
  KeyLoad r;
  if constexpr (F32) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(keys) +
                                                     (slot0 + (lane >> 3)) * kIdxDim + 8 * (lane & 7));
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  } else {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(keys) +
                                                     (slot0 + (lane >> 3)) * kIdxDim + 8 * (lane & 7));
    r.a = __builtin_nontemporal_load(p);
    r.b = u32x4{0, 0, 0, 0};
  }
  return r;
}

template <bool F32>
__device__ __forceinline__ float unit_score(const KeyLoad &k, const float (&q)[8]) {
  float s;
  if constexpr (F32) {
    s = q[0] * __uint_as_float(k.a[0]);
    s = fmaf(q[1], __uint_as_float(k.a[1]), s);
    s = fmaf(q[2], __uint_as_float(k.a[2]), s);
    s = fmaf(q[3], __uint_as_float(k.a[3]), s);
    s = fmaf(q[4], __uint_as_float(k.b[0]), s);
    s = fmaf(q[5], __uint_as_float(k.b[1]), s);
    s = fmaf(q[6], __uint_as_float(k.b[2]), s);
    s = fmaf(q[7], __uint_as_float(k.b[3]), s);
  } else {
    s = q[0] * __uint_as_float(k.a[0] << 16);
    s = fmaf(q[1], __uint_as_float(k.a[0] & 0xFFFF0000u), s);
    s = fmaf(q[2], __uint_as_float(k.a[1] << 16), s);
    s = fmaf(q[3], __uint_as_float(k.a[1] & 0xFFFF0000u), s);
    s = fmaf(q[4], __uint_as_float(k.a[2] << 16), s);
    s = fmaf(q[5], __uint_as_float(k.a[2] & 0xFFFF0000u), s);
    s = fmaf(q[6], __uint_as_float(k.a[3] << 16), s);
    s = fmaf(q[7], __uint_as_float(k.a[3] & 0xFFFF0000u), s);
  }
  return group8_sum(s);
}

// ---- multi-head FP4 keys: 32 query heads x 128 dims on v_mfma_f32_32x32x16_f16
// One tile = 32 positions x 32 heads.  Lane l works on position l % 32 of the
// tile and half h = l / 32 of the key: dims 64 h .. 64 h + 63 (32 nibble bytes
// and 4 E4M3 scales).  The contraction's 16-wide k-step ks pairs dims
// 64 h + 8 ks .. + 7 of both halves, for the query (A, row = head) and the key
// (B, column = position) alike, so every lane dequantizes only its own bytes.
// D lane l holds heads 8 (e / 4) + 4 h + e % 4 (e < 16) of position l % 32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kFp4IdxDim = 128;
constexpr int kFp4IdxMaxHeads = 32;

enum KeyFmt { kKeyBf16 = 0, kKeyF32 = 1, kKeyFp4 = 2 };

struct Fp4Half {
  u32x4 c0, c1;  // 64 nibbles
  uint32_t sc;   // 4 scales
};

__device__ __forceinline__ Fp4Half load_fp4_half(const KvLayerDev &L, int64_t slot, int lane) {
  const int h = lane >> 5;
  const u32x4 *cp =
      reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(L.idx_keys) + slot * (kFp4IdxDim / 2) + 32 * h);
  Fp4Half r;
  r.c0 = __builtin_nontemporal_load(cp);
  r.c1 = __builtin_nontemporal_load(cp + 1);
  r.sc = __builtin_nontemporal_load(
      reinterpret_cast<const uint32_t *>(L.idx_scales + slot * (kFp4IdxDim / kGroup) + 4 * h));
  return r;
}

struct Fp4Query {
  f16x8 qa[8];   // this lane's head row (lane % 32), dims 64 h + 8 ks .. + 7
  float wr[16];  // weights of the 16 heads this lane's results hold (0 past the heads)
};

__device__ __forceinline__ void load_fp4_query(IdxQuery q, int b, int heads, int lane, Fp4Query &Q) {
  const int r = lane & 31, h = lane >> 5;
  const f16 *qrow = static_cast<const f16 *>(q.q) + ((size_t)b * heads + (r < heads ? r : 0)) * kFp4IdxDim + 64 * h;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const f16x8 v = *reinterpret_cast<const f16x8 *>(qrow + 8 * ks);
    Q.qa[ks] = r < heads ? v : f16x8{};
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {  // unconditional (clamped) loads, masked after
    const int row = 8 * (e >> 2) + 4 * h + (e & 3);
    const float w = q.w[(size_t)b * heads + (row < heads ? row : heads - 1)];
    Q.wr[e] = row < heads ? w : 0.0f;
  }
}

// Score of this lane's position: sum over heads of w * max(0, q . k) (both
// lanes of a position return it).
__device__ __forceinline__ float fp4_tile_score(const Fp4Half &k, const Fp4Query &Q) {
  const uint32_t words[8] = {k.c0[0], k.c0[1], k.c0[2], k.c0[3], k.c1[0], k.c1[1], k.c1[2], k.c1[3]};
  const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.sc, 1.0f, false);
  const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.sc, 1.0f, true);
  const f16 sc[4] = {s01[0], s01[1], s23[0], s23[1]};
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Q.qa[ks], deq8(words[ks], sc[ks >> 1]), acc, 0, 0, 0);
  // max(x, 0) as the signed-integer maximum of the fp32 bits (negative values
  // and -0 have the sign bit set, so they become +0): one instruction, where
  // fmaxf also canonicalizes its input
  // four independent partial sums instead of one chain of 16 dependent FMAs
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int e = 0; e < 16; ++e)
    part[e & 3] = fmaf(Q.wr[e], __int_as_float(max(__float_as_int(acc[e]), 0)), part[e & 3]);
  const float s = (part[0] + part[1]) + (part[2] + part[3]);
  return s + __shfl_xor(s, 32);
}

__device__ __forceinline__ int row_len(const SeqsDev &S, int b) {
  const int n = S.seq_lens[b];
  return n < 0 ? 0 : (n > S.max_len ? S.max_len : n);
}

// Physical block of page `page` of row b, or -1 when it is not mapped.
__device__ __forceinline__ int page_block(const SeqsDev &S, int num_blocks, int b, int64_t page) {
  if (page < 0 || page >= S.max_blocks) return -1;
  const int blk = S.block_table[(int64_t)b * S.max_blocks + page];
  return (blk >= 0 && blk < num_blocks) ? blk : -1;
}

// ------------------------------------------------------------------ block-wide helpers
// Exclusive prefix sum of one value per thread across a workgroup of NT
// threads.  Returns the prefix; *total gets the sum.  scratch: NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch, uint32_t *total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t wave_base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = scratch[w];
    wave_base += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return wave_base + incl - v;
}

// Threshold digit of a 2048-bin histogram in LDS, computed by one wave:
// the bin d with sum(hist[d+1..]) < need <= sum(hist[d..]).  Result in
// res[0] = d, res[1] = sum(hist[d+1..]), res[2] = found (0 when all bins hold
// fewer than `need`; then d = 0 and res[1] = total - hist[0]).  All 64 lanes
// of the calling wave take part; the caller synchronizes before reading res.
__device__ __forceinline__ void find_threshold_wave(const uint32_t *hist, uint32_t need, uint32_t *res) {
  const int t = threadIdx.x & 63;
  {
    constexpr int per = kBins / 64;  // lane l owns bins [32l, 32l+32)
    const u32x4 *h4 = reinterpret_cast<const u32x4 *>(&hist[per * t]);
    u32x4 v[per / 4];
#pragma unroll
    for (int j = 0; j < per / 4; ++j) v[j] = h4[j];
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < per / 4; ++j) mine += v[j][0] + v[j][1] + v[j][2] + v[j][3];
    const uint32_t pre = wave_inclusive_sum(mine);  // lanes 0..t
    const uint32_t total = wave_last(pre);
    const uint32_t above_me = total - pre;  // lanes above t
    const uint64_t hit = __ballot(above_me < need && above_me + mine >= need);
    if (hit) {
      // the boundary bin is one of lane src's: lanes 0..31 take its bins from
      // the top down and a prefix sum over lanes gives each bin's count above
      const int src = __ffsll((unsigned long long)hit) - 1;
      const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)above_me, src);
      const int bin = per * src + (per - 1) - (t & (per - 1));
      const uint32_t h = t < per ? hist[bin] : 0u;
      const uint32_t cum = wave_inclusive_sum(h);
      const uint64_t q = __ballot(t < per && base + cum - h < need && base + cum >= need);
      if (t == __ffsll((unsigned long long)q) - 1) {
        res[0] = (uint32_t)bin;
        res[1] = base + cum - h;
        res[2] = 1u;
      }
    } else if (t == 0) {
      res[0] = 0u;
      res[1] = total - hist[0];
      res[2] = 0u;
    }
  }
}

// The same search run by wave 0, followed by a barrier (every thread calls it).
__device__ __forceinline__ void find_threshold(const uint32_t *hist, uint32_t need, uint32_t *res) {
  if (threadIdx.x < 64) find_threshold_wave(hist, need, res);
  __syncthreads();
}

// Ordered compaction over a workgroup of NT threads.  Wave w owns items
// [64 IPT w, 64 IPT (w + 1)); its lane l holds items 64 IPT w + 64 j + l
// (j < IPT), so item order is (wave, j, lane) order.  Bit j of flags keeps
// item j of this lane; emit(j, slot, keep) is called for every item, and for
// a kept one slot = base + (kept items before it).  Returns the number kept.
// red: NT/64 words of LDS.
template <int NT, int IPT, class Emit>
__device__ __forceinline__ uint32_t ordered_emit(uint32_t flags, uint32_t *red, uint32_t base, Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = __lanemask_lt();
  uint64_t bal[IPT];
  uint32_t wtot = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    bal[j] = __ballot((flags >> j) & 1u);
    wtot += (uint32_t)__popcll(bal[j]);
  }
  if (lane == 0) red[wave] = wtot;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = red[w];
    wbase += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  uint32_t run = base + wbase;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    emit(j, run + (uint32_t)__popcll(bal[j] & below), ((flags >> j) & 1u) != 0u);
    run += (uint32_t)__popcll(bal[j]);
  }
  return tot;
}

// ------------------------------------------------------------------ producer: emission
// Emits the best items of a producer workgroup (keys in LDS, key 0 = no item)
// as an ordered candidate segment of at most `cap` items: whole 11-bit key
// bins from the top, then the best 11-bit sub-bins of the boundary bin.
// Lane l of wave w owns items 64 IPT w + 64 j + l; pos_of(i) is item i's
// position.
// Zeroes NH histograms of kBins words with a 256-thread workgroup.
template <int NH>
__device__ __forceinline__ void zero_hists(uint32_t (*hist)[kBins]) {
  u32x4 *h4 = reinterpret_cast<u32x4 *>(&hist[0][0]);
#pragma unroll
  for (int i = 0; i < NH * kBins / 4 / 256; ++i) h4[256 * i + threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
}

// Absolute digits (the key's top 11 bits, then the next 11 inside the
// boundary bin).  hist[0], hist[1]: level-1 and level-2 histograms, zeroed by
// the caller before a barrier that precedes the call (zero_hists).
template <int NT, int IPT, class PosOf>
__device__ __forceinline__ void emit_segment_abs(const uint32_t *keys_l, int cap, uint2 *cand_seg, SegInfo *info,
                                                 uint32_t (*hist)[kBins], uint32_t *red, PosOf pos_of) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i0 = 64 * IPT * wave + lane;  // this lane's items: i0 + 64 j
  uint32_t k[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) k[j] = keys_l[i0 + 64 * j];
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if (k[j]) atomicAdd(&hist[0][k[j] >> 21], 1u);
  __syncthreads();
  find_threshold(hist[0], (uint32_t)cap + 1u, red + 16);
  const uint32_t d1 = red[16], above = red[17];
  const bool cut = red[18] != 0u;
  uint32_t d2 = 0, edge = 0;
  if (cut) {
    // level 2 inside the boundary bin d1: room for cap - above of its items
    const uint32_t room = (uint32_t)cap - above;
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (k[j] && (k[j] >> 21) == d1) atomicAdd(&hist[1][(k[j] >> 10) & 0x7FFu], 1u);
    __syncthreads();
    find_threshold(hist[1], room + 1u, red + 16);
    d2 = red[16];  // found: bin d1 holds more than `room` items
    const uint64_t e = ((uint64_t)d1 << 21) + ((uint64_t)(d2 + 1u) << 10);
    edge = e > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)e;
  }
  uint32_t flags = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const uint32_t key = k[j];
    const bool em =
        key != 0u && (!cut || (key >> 21) > d1 || ((key >> 21) == d1 && ((key >> 10) & 0x7FFu) > d2));
    flags |= em ? (1u << j) : 0u;
  }
  const uint32_t total = ordered_emit<NT, IPT>(flags, red, 0u, [&](int j, uint32_t slot, bool keep) {
    if (keep) cand_seg[slot] = make_uint2(k[j], pos_of(i0 + 64 * j));
  });
  for (int i = (int)total + t; i < cap; i += NT) cand_seg[i] = make_uint2(0u, 0u);  // unused slots: no item
  if (t == 0) *info = SegInfo{total, edge};
}

// Both segments of a hierarchical scan workgroup at once (positions: 256 IPT
// keys, IPT per thread; blocks: 32 IPT keys, one per thread of the first
// 32 IPT), with the same cut rule as emit_segment: the two histograms share
// each barrier and their threshold searches run side by side in waves 0 and
// 1.
// hist[0..3]: level-1 and level-2 histograms of positions and blocks, zeroed
// by the caller before a barrier that precedes the call.
template <int IPT, class PosP, class PosB>
__device__ __forceinline__ void emit_segment_pair_abs(const uint32_t *pkeys, int cap_p, uint2 *cand_p,
                                                      SegInfo *info_p, PosP pos_p, const uint32_t *bkeys, int cap_b,
                                                      uint2 *cand_b, SegInfo *info_b, PosB pos_b,
                                                      uint32_t (*hist)[kBins], uint32_t *red) {
  constexpr int NT = 256;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ip0 = 64 * IPT * wave + lane, ib = 64 * wave + lane;
  uint32_t *hist_p = hist[0], *hist_b = hist[1];
  uint32_t kp[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) kp[j] = pkeys[ip0 + 64 * j];
  const uint32_t kb = ib < 32 * IPT ? bkeys[ib] : 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    if (kp[j]) atomicAdd(&hist_p[kp[j] >> 21], 1u);
  if (kb) atomicAdd(&hist_b[kb >> 21], 1u);
  __syncthreads();
  if (wave == 0) find_threshold_wave(hist_p, (uint32_t)cap_p + 1u, red + 16);
  if (wave == 1) find_threshold_wave(hist_b, (uint32_t)cap_b + 1u, red + 20);
  __syncthreads();
  const uint32_t d1p = red[16], above_p = red[17], d1b = red[20], above_b = red[21];
  const bool cut_p = red[18] != 0u, cut_b = red[22] != 0u;
  uint32_t d2p = 0, d2b = 0, edge_p = 0, edge_b = 0;
  if (cut_p || cut_b) {
    // level 2 inside each boundary bin d1: room for cap - above of its items
    hist_p = hist[2];
    hist_b = hist[3];
    if (cut_p) {
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if (kp[j] && (kp[j] >> 21) == d1p) atomicAdd(&hist_p[(kp[j] >> 10) & 0x7FFu], 1u);
    }
    if (cut_b && kb && (kb >> 21) == d1b) atomicAdd(&hist_b[(kb >> 10) & 0x7FFu], 1u);
    __syncthreads();
    if (wave == 0 && cut_p) find_threshold_wave(hist_p, (uint32_t)cap_p - above_p + 1u, red + 16);
    if (wave == 1 && cut_b) find_threshold_wave(hist_b, (uint32_t)cap_b - above_b + 1u, red + 20);
    __syncthreads();
    if (cut_p) {
      d2p = red[16];
      const uint64_t e = ((uint64_t)d1p << 21) + ((uint64_t)(d2p + 1u) << 10);
      edge_p = e > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)e;
    }
    if (cut_b) {
      d2b = red[20];
      const uint64_t e = ((uint64_t)d1b << 21) + ((uint64_t)(d2b + 1u) << 10);
      edge_b = e > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)e;
    }
  }
  auto emit = [](uint32_t key, bool cut, uint32_t d1, uint32_t d2) {
    return key != 0u && (!cut || (key >> 21) > d1 || ((key >> 21) == d1 && ((key >> 10) & 0x7FFu) > d2));
  };
  // ordered compaction of both segments with one exchange of wave totals
  const uint64_t below = __lanemask_lt();
  uint64_t bal[IPT];
  uint32_t wtot_p = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    bal[j] = __ballot(emit(kp[j], cut_p, d1p, d2p));
    wtot_p += (uint32_t)__popcll(bal[j]);
  }
  const bool keep_b = emit(kb, cut_b, d1b, d2b);
  const uint64_t bal_b = __ballot(keep_b);
  if (lane == 0) {
    red[wave] = wtot_p;
    red[4 + wave] = (uint32_t)__popcll(bal_b);
  }
  __syncthreads();
  uint32_t run = 0, total_p = 0, slot_b = 0, total_b = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t xp = red[w], xb = red[4 + w];
    run += w < wave ? xp : 0u;
    slot_b += w < wave ? xb : 0u;
    total_p += xp;
    total_b += xb;
  }
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((bal[j] >> lane) & 1u) cand_p[run + (uint32_t)__popcll(bal[j] & below)] = make_uint2(kp[j], pos_p(ip0 + 64 * j));
    run += (uint32_t)__popcll(bal[j]);
  }
  if (keep_b) cand_b[slot_b + (uint32_t)__popcll(bal_b & below)] = make_uint2(kb, pos_b(ib));
  for (int i = (int)total_p + t; i < cap_p; i += NT) cand_p[i] = make_uint2(0u, 0u);  // unused slots: no item
  for (int i = (int)total_b + t; i < cap_b; i += NT) cand_b[i] = make_uint2(0u, 0u);
  if (t == 0) {
    *info_p = SegInfo{total_p, edge_p};
    *info_b = SegInfo{total_b, edge_b};
  }
}

// Relative digits.  Bin of a key below the segment's largest key M: bins of
// 2^12 key units counted down from M (bin 2047 holds M); keys 2047 or more
// bins below M are "far" (bin 0) and are only counted, not binned.  Keys are
// order-preserving images of fp32 scores, close to logarithmic in the score,
// so the window spans about a factor of 2 below the largest score at any
// scale, which holds a segment's best few items for the score distributions
// of an indexer, at 2^12-unit resolution.  The cut keeps whole bins from the
// top (at most cap items); everything left has a key below the edge.  When
// the window holds fewer than cap items and far items remain, the absolute
// two-level emission runs instead (it can use more of the budget there).
constexpr int kRelShift = 12;
// The relative digits are used when the budget is a small share of the
// segment (at most 1/50 of its items, e.g. 12 of 2048 at 1M positions);
// larger budgets reach further below the maximum than the window does for
// Gaussian-like scores and go straight to the absolute emission.
__device__ __forceinline__ bool rel_fits(int cap, int items) { return 50 * cap <= items; }
template <int SH = kRelShift>
__device__ __forceinline__ uint32_t rel_bin(uint32_t key, uint32_t m) {
  const uint32_t d = (m - key) >> SH;
  return d >= (uint32_t)(kBins - 1) ? 0u : (uint32_t)(kBins - 1) - d;
}
// Every key in bins <= d is below this (a key of bin d > 0 is at most
// M - (2047 - d) 2^12; a far key at most M - 2047 2^12; both >= 1 when such
// a key exists).
template <int SH = kRelShift>
__device__ __forceinline__ uint32_t rel_edge(uint32_t m, uint32_t d) {
  return m - (((uint32_t)(kBins - 1) - d) << SH) + 1u;
}

// Relative-digit histogram of one lane's keys (far keys only counted) and
// its wave's count of far keys in far_w[wave] (0 or the count; lane 0 writes).
template <int IPT, int SH = kRelShift>
__device__ __forceinline__ void rel_hist(const uint32_t (&k)[IPT], uint32_t m, uint32_t *hist, uint32_t *far_w) {
  uint32_t far = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const uint32_t bin = rel_bin<SH>(k[j], m);
    const bool is_far = k[j] != 0u && bin == 0u;
    far += (uint32_t)__popcll(__ballot(is_far));
    if (k[j] != 0u && bin != 0u) atomicAdd(&hist[bin], 1u);
  }
  if ((threadIdx.x & 63) == 0) far_w[threadIdx.x >> 6] = far;
}

// The cut of one relative-digit segment from its threshold search (for
// cap + 1 over the binned keys) and its far count: returns false when the
// absolute emission must run instead; else *cut / *d say which bins are kept
// (all when !cut, else bins > d) and *edge the segment's edge.
template <int SH = kRelShift>
__device__ __forceinline__ bool rel_cut(const uint32_t *res, uint32_t far, int cap, uint32_t m, bool *cut,
                                        uint32_t *d, uint32_t *edge) {
  const bool found = res[2] != 0u;
  if (found) {  // the boundary lies in the window (bin >= 1)
    *cut = true;
    *d = res[0];
    *edge = rel_edge<SH>(m, res[0]);
    return true;
  }
  const uint32_t binned = res[1];  // total of bins 1 .. 2047 (bin 0 is never binned)
  if (far == 0u) {                 // everything fits
    *cut = false;
    *d = 0u;
    *edge = 0u;
    return true;
  }
  if (binned == (uint32_t)cap) {  // exactly the budget in the window, the rest far
    *cut = true;
    *d = 0u;
    *edge = rel_edge<SH>(m, 0u);
    return true;
  }
  return false;
}

// Largest of this lane's keys over the workgroup (every thread gets it).
// red: NT/64 words; ends with a barrier.
template <int NT, int IPT>
__device__ __forceinline__ uint32_t block_max_key(const uint32_t (&k)[IPT], uint32_t *red) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) m = max(m, k[j]);
  m = wave_last(wave_inclusive_max(m));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  uint32_t r = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) r = max(r, red[w]);
  return r;
}

// emit_segment with relative digits below a known largest key m of the
// segment's keys (same contract as emit_segment_abs; hist[0], hist[1] zeroed
// by the caller before a barrier that precedes the call; red: NT/64 + 24
// words).
template <int NT, int IPT, int SH = kRelShift, class PosOf>
__device__ __forceinline__ void emit_segment_m(uint32_t m, const uint32_t *keys_l, int cap, uint2 *cand_seg,
                                               SegInfo *info, uint32_t (*hist)[kBins], uint32_t *red,
                                               PosOf pos_of) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i0 = 64 * IPT * wave + lane;  // this lane's items: i0 + 64 j
  if (!rel_fits(cap, NT * IPT)) {  // uniform
    emit_segment_abs<NT, IPT>(keys_l, cap, cand_seg, info, hist, red, pos_of);
    return;
  }
  uint32_t k[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) k[j] = keys_l[i0 + 64 * j];
  rel_hist<IPT, SH>(k, m, hist[0], red + 24 - NW);
  __syncthreads();
  find_threshold(hist[0], (uint32_t)cap + 1u, red + 16);
  uint32_t far = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) far += red[24 - NW + w];
  bool cut;
  uint32_t d1, edge;
  if (!rel_cut<SH>(red + 16, far, cap, m, &cut, &d1, &edge)) {  // uniform
    zero_hists<1>(hist);
    __syncthreads();
    emit_segment_abs<NT, IPT>(keys_l, cap, cand_seg, info, hist, red, pos_of);
    return;
  }
  uint32_t flags = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool em = k[j] != 0u && (!cut || rel_bin<SH>(k[j], m) > d1);
    flags |= em ? (1u << j) : 0u;
  }
  const uint32_t total = ordered_emit<NT, IPT>(flags, red, 0u, [&](int j, uint32_t slot, bool keep) {
    if (keep) cand_seg[slot] = make_uint2(k[j], pos_of(i0 + 64 * j));
  });
  for (int i = (int)total + t; i < cap; i += NT) cand_seg[i] = make_uint2(0u, 0u);  // unused slots: no item
  if (t == 0) *info = SegInfo{total, edge};
}

// The same, finding the largest key first (one more barrier).
template <int NT, int IPT, class PosOf>
__device__ __forceinline__ void emit_segment(const uint32_t *keys_l, int cap, uint2 *cand_seg, SegInfo *info,
                                             uint32_t (*hist)[kBins], uint32_t *red, PosOf pos_of) {
  if (!rel_fits(cap, NT * IPT)) {  // uniform
    emit_segment_abs<NT, IPT>(keys_l, cap, cand_seg, info, hist, red, pos_of);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t k[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) k[j] = keys_l[64 * IPT * wave + lane + 64 * j];
  const uint32_t m = block_max_key<NT, IPT>(k, red + 8);
  emit_segment_m<NT, IPT>(m, keys_l, cap, cand_seg, info, hist, red, pos_of);
}

// emit_segment_pair with relative digits below m, the largest position key
// (which is also the largest block key): both histograms and both threshold
// searches (waves 0 and 1) share their barriers.  hist[0..3] zeroed by the
// caller before a barrier that precedes the call; red: 36 words.
template <int IPT, int SH, class PosP, class PosB>
__device__ __forceinline__ void emit_segment_pair(uint32_t m, const uint32_t *pkeys, int cap_p, uint2 *cand_p,
                                                  SegInfo *info_p, PosP pos_p, const uint32_t *bkeys, int cap_b,
                                                  uint2 *cand_b, SegInfo *info_b, PosB pos_b,
                                                  uint32_t (*hist)[kBins], uint32_t *red) {
  constexpr int NT = 256;
  // (a block key is the largest of its 8 positions: the best blocks' keys are
  // among the best positions' keys, so blocks are measured against positions)
  if (!rel_fits(cap_p, NT * IPT) || !rel_fits(cap_b, NT * IPT)) {  // uniform
    emit_segment_pair_abs<IPT>(pkeys, cap_p, cand_p, info_p, pos_p, bkeys, cap_b, cand_b, info_b, pos_b, hist, red);
    return;
  }
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ip0 = 64 * IPT * wave + lane, ib = 64 * wave + lane;
  uint32_t kp[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) kp[j] = pkeys[ip0 + 64 * j];
  const uint32_t kb1[1] = {ib < 32 * IPT ? bkeys[ib] : 0u};
  const uint32_t kb = kb1[0];
  const uint32_t mp = m, mb = m;
  rel_hist<IPT, SH>(kp, mp, hist[0], red + 24);
  rel_hist<1, SH>(kb1, mb, hist[1], red + 28);
  __syncthreads();
  if (wave == 0) find_threshold_wave(hist[0], (uint32_t)cap_p + 1u, red + 16);
  if (wave == 1) find_threshold_wave(hist[1], (uint32_t)cap_b + 1u, red + 20);
  __syncthreads();
  uint32_t far_p = 0u, far_b = 0u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    far_p += red[24 + w];
    far_b += red[28 + w];
  }
  bool cut_p, cut_b;
  uint32_t d1p, d1b, edge_p, edge_b;
  const bool ok_p = rel_cut<SH>(red + 16, far_p, cap_p, mp, &cut_p, &d1p, &edge_p);
  const bool ok_b = rel_cut<SH>(red + 20, far_b, cap_b, mb, &cut_b, &d1b, &edge_b);
  if (!ok_p || !ok_b) {  // uniform: the absolute emission for both
    __syncthreads();     // every thread has read red[]
    zero_hists<2>(hist);
    __syncthreads();
    emit_segment_pair_abs<IPT>(pkeys, cap_p, cand_p, info_p, pos_p, bkeys, cap_b, cand_b, info_b, pos_b, hist, red);
    return;
  }
  // ordered compaction of both segments with one exchange of wave totals
  const uint64_t below = __lanemask_lt();
  uint64_t bal[IPT];
  uint32_t wtot_p = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    bal[j] = __ballot(kp[j] != 0u && (!cut_p || rel_bin<SH>(kp[j], mp) > d1p));
    wtot_p += (uint32_t)__popcll(bal[j]);
  }
  const bool keep_b = kb != 0u && (!cut_b || rel_bin<SH>(kb, mb) > d1b);
  const uint64_t bal_b = __ballot(keep_b);
  if (lane == 0) {  // (red[0..7] is free here: the values read above live in red[8..31])
    red[wave] = wtot_p;
    red[4 + wave] = (uint32_t)__popcll(bal_b);
  }
  __syncthreads();
  uint32_t run = 0, total_p = 0, slot_b = 0, total_b = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t xp = red[w], xb = red[4 + w];
    run += w < wave ? xp : 0u;
    slot_b += w < wave ? xb : 0u;
    total_p += xp;
    total_b += xb;
  }
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((bal[j] >> lane) & 1u) cand_p[run + (uint32_t)__popcll(bal[j] & below)] = make_uint2(kp[j], pos_p(ip0 + 64 * j));
    run += (uint32_t)__popcll(bal[j]);
  }
  if (keep_b) cand_b[slot_b + (uint32_t)__popcll(bal_b & below)] = make_uint2(kb, pos_b(ib));
  for (int i = (int)total_p + t; i < cap_p; i += NT) cand_p[i] = make_uint2(0u, 0u);  // unused slots: no item
  for (int i = (int)total_b + t; i < cap_b; i += NT) cand_b[i] = make_uint2(0u, 0u);
  if (t == 0) {
    *info_p = SegInfo{total_p, edge_p};
    *info_b = SegInfo{total_b, edge_b};
  }
}

// ------------------------------------------------------------------ producer: full scan
struct ScanArgs {
  KvLayerDev L;
  SeqsDev S;
  IdxQuery q;
  int K, P;  // top-K, pool blocks (hierarchical)
  SelWs w;
  // Rows appended in the same launch (workgroups x >= scan_wgs, one per
  // append and sequence) at position seq_lens[b] - 1.  When one of them
  // writes the scanned keys, new_key is its key input: the scan workgroup
  // covering that position scores it from there (the cache row may not be
  // written yet).
  int scan_wgs, n_app;
  AppendRow app[kMaxAppendRows];
  const void *new_key;
  uint32_t *dbg;  // debug flag word, or null
};

// SLICE: positions per workgroup (segment), 2048 or 1024.
template <int KF, bool HIER, int SLICE>
__global__ void __launch_bounds__(256) scan_kernel(ScanArgs a) {
  constexpr bool F32 = KF == kKeyF32;
  constexpr int kPages = SLICE / kPage;   // 32 or 16
  constexpr int kPagesPerWave = kPages / 4;
  constexpr int kBlocks = SLICE / kBlk;   // 256 or 128
  constexpr int kIpt = SLICE / 256;       // positions per thread in the emission
  // relative-digit emission (the slice's largest key tracked while scoring);
  // the FP4 multi-head scores (weighted sums of ReLUs) spread further below
  // the slice maximum than a dot product's, so their bins are 4x wider (the
  // window spans 4 binades instead of 1)
  constexpr bool kRel = true;
  constexpr int kSh = KF == kKeyFp4 ? kRelShift + 2 : kRelShift;
  __shared__ int32_t pg[kPages];
  __shared__ __attribute__((aligned(16))) uint32_t pkey[SLICE];
  __shared__ __attribute__((aligned(16))) uint32_t bkey[kBlocks];
  // histograms of the emission: positions (level 1, 2) and, hierarchical,
  // blocks (level 1, 2); zeroed while the first loads are in flight
  __shared__ __attribute__((aligned(16))) uint32_t hist[HIER ? 4 : 2][kBins];
  __shared__ uint32_t red[36];
  __shared__ uint32_t kmax_l;  // largest key of the segment (LDS atomic max of the waves' maxima)
  const int b = blockIdx.y, wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wg >= a.scan_wgs) {  // an append workgroup (uniform)
    const AppendRow &r = a.app[wg - a.scan_wgs];
    if (tid < 64) append_row(r.L, a.S, b, -1, r.latent, r.rope, r.idx_key, tid, a.dbg);
    return;
  }
  // this slice's page-table entries are read together with the length (one
  // memory round trip before the key loads instead of two); entries of pages
  // past the length are masked below
  int blk_raw = -1;
  if (tid < kPages) {
    const int64_t page = (int64_t)wg * kPages + tid;
    if (page < a.S.max_blocks) blk_raw = a.S.block_table[(int64_t)b * a.S.max_blocks + page];
  }
  const int sl = a.S.seq_lens[b];  // read once: a reload after the key loads would cost a memory round trip
  const int n = sl < 0 ? 0 : (sl > a.S.max_len ? a.S.max_len : sl);
  const int64_t base = (int64_t)wg * SLICE;
  if (a.dbg != nullptr && wg == 0 && tid == 0 && (sl < 0 || sl > a.S.max_len)) dbg_raise(a.dbg, kDbgSeqLen);
  if (base >= n) return;  // segments past the row are never read
  zero_hists<HIER ? 4 : 2>(hist);
  if (tid == 0) kmax_l = 0u;
  uint32_t kmax = 0u;  // this lane's largest key
  const bool can_load = a.L.num_blocks > 0;  // an empty pool: every page is unmapped
  if (tid < kPages) {
    pg[tid] = (base + 64 * tid < n && blk_raw >= 0 && blk_raw < a.L.num_blocks) ? blk_raw : -1;
    if (a.dbg != nullptr && base + 64 * tid < n && pg[tid] < 0) dbg_raise(a.dbg, kDbgPage);
  }
  float q[8];
  Fp4Query Q;
  if constexpr (KF == kKeyFp4) {
    load_fp4_query(a.q, b, a.L.idx_heads, lane, Q);
  } else {
    const float *qp = static_cast<const float *>(a.q.q) + (size_t)b * kIdxDim + 8 * (lane & 7);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = qp[e];
  }
  __syncthreads();
  // wave w streams pages w, w+4, .., w+28 (the workgroup's four waves read
  // four neighbouring pages at a time), one page at a time (8 loads of 1 KB,
  // or for FP4 keys two tiles of 32 positions) with the next page's loads in
  // flight
  constexpr int kDepth = 2;  // pages whose loads are in flight (deeper measured slower, also at one workgroup per CU)
  if constexpr (KF == kKeyFp4) {
    if (can_load) {
      Fp4Half kt[kDepth][2];
      auto issue4 = [&](int pp, Fp4Half(&dst)[2]) {
        const int pid = pg[4 * pp + wave];
        const int64_t s0 = (int64_t)(pid < 0 ? 0 : pid) * kPage;  // unmapped: read slot 0, masked below
#pragma unroll
        for (int j = 0; j < 2; ++j) dst[j] = load_fp4_half(a.L, s0 + 32 * j + (lane & 31), lane);
      };
      issue4(0, kt[0]);
#pragma unroll
      for (int pp = 0; pp < kPagesPerWave; ++pp) {
        if (pp + 1 < kPagesPerWave) issue4(pp + 1, kt[(pp + 1) % kDepth]);
        const int page = 4 * pp + wave;
        const bool mapped = pg[page] >= 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int lp = page * kPage + 32 * j + (lane & 31);  // local position
          const float sc = fp4_tile_score(kt[pp % kDepth][j], Q);
          const uint32_t key = (mapped && base + lp < n) ? score_key(sc) : 0u;
          kmax = max(kmax, key);
          if (lane < 32) pkey[lp] = key;
        }
      }
    } else {
      for (int i = tid; i < SLICE; i += 256) pkey[i] = 0u;
    }
  } else {
  KeyLoad kl[kDepth][8];
  auto issue = [&](int pp, KeyLoad(&dst)[8]) {
    const int pid = pg[4 * pp + wave];
    const int id = pid < 0 ? 0 : pid;  // unmapped: read slot 0, masked below
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[u] = load_unit<F32>(a.L.idx_keys, (int64_t)id * kPage + 8 * u, lane);
  };
  if (can_load) {
#pragma unroll
    for (int pp = 0; pp < kDepth - 1; ++pp) issue(pp, kl[pp]);
#pragma unroll
    for (int pp = 0; pp < kPagesPerWave; ++pp) {
      if (pp + kDepth - 1 < kPagesPerWave) issue(pp + kDepth - 1, kl[(pp + kDepth - 1) % kDepth]);
      const int page = 4 * pp + wave;
      const bool mapped = pg[page] >= 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int lp = page * kPage + 8 * u + (lane >> 3);  // local position
        const float sc = unit_score<F32>(kl[pp % kDepth][u], q);
        const uint32_t key = (mapped && base + lp < n) ? score_key(sc) : 0u;
        kmax = max(kmax, key);
        if ((lane & 7) == 0) pkey[lp] = key;
      }
    }
  } else {
    for (int i = tid; i < SLICE; i += 256) pkey[i] = 0u;
  }
  }
  if constexpr (kRel) {
    kmax = wave_last(wave_inclusive_max(kmax));
    if (lane == 0) atomicMax(&kmax_l, kmax);
  }
  __syncthreads();
  if (a.new_key != nullptr && sl - 1 >= base && sl - 1 < base + SLICE &&
      sl <= n) {  // uniform: this workgroup holds the appended position
    const int lp = sl - 1 - (int)base;
    if (wave == 0 && pg[lp / kPage] >= 0) {
      // the same lane layout and arithmetic as the streaming loop, on the input key
      if constexpr (KF == kKeyFp4) {
        Fp4Half kh = Fp4Half{u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, 0u};
        if ((lane & 31) == (lp & 31)) {
          const float *src = static_cast<const float *>(a.new_key) + (size_t)b * kFp4IdxDim + 64 * (lane >> 5);
          uint32_t wd[8], sc = 0;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = src[16 * g + i];
            sc |= pack_group16(v, &wd[2 * g], &wd[2 * g + 1]) << (8 * g);
          }
          kh = Fp4Half{u32x4{wd[0], wd[1], wd[2], wd[3]}, u32x4{wd[4], wd[5], wd[6], wd[7]}, sc};
        }
        const float sc = fp4_tile_score(kh, Q);
        if (lane == (lp & 31)) {
          pkey[lp] = score_key(sc);
          atomicMax(&kmax_l, score_key(sc));
        }
      } else {
        KeyLoad kl;
        if constexpr (F32) {
          const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(a.new_key) +
                                                           (size_t)b * kIdxDim + 8 * (lane & 7));
          kl = KeyLoad{p[0], p[1]};
        } else {
          const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.new_key) +
                                                           (size_t)b * kIdxDim + 8 * (lane & 7));
          kl = KeyLoad{p[0], u32x4{0, 0, 0, 0}};
        }
        const float sc = unit_score<F32>(kl, q);
        if (lane == 0) {
          pkey[lp] = score_key(sc);
          atomicMax(&kmax_l, score_key(sc));
        }
      }
    }
    __syncthreads();
  }
  if constexpr (HIER) {
    // block key = largest key of its 8 positions (unmapped or past-the-end positions hold key 0)
    if (tid < kBlocks) {
      const u32x4 *p4 = reinterpret_cast<const u32x4 *>(pkey + kBlk * tid);
      const u32x4 x = p4[0], y = p4[1];
      uint32_t m = max(max(max(x[0], x[1]), max(x[2], x[3])), max(max(y[0], y[1]), max(y[2], y[3])));
      bkey[tid] = m;  // (read back only by this thread: the key store and the emission's block item tid)
    }
  }
  // store every key (the select re-reads segments that overflow their budget)
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(pkey);
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.w.keys + (size_t)b * a.w.cap_keys + base);
#pragma unroll
    for (int i = 0; i < SLICE / 4 / 256; ++i) dst[tid + 256 * i] = src[tid + 256 * i];
    if constexpr (HIER) {
      if (tid < kBlocks) a.w.bkeys[(size_t)b * a.w.cap_blocks + base / kBlk + tid] = bkey[tid];
    }
  }
  const int nseg = (n + SLICE - 1) / SLICE;
  const int cap = seg_budget(a.K, nseg, SLICE);
  if constexpr (HIER) {
    const int cap_b = seg_budget(a.P, nseg, kBlocks);
    if constexpr (kRel) {
      emit_segment_pair<kIpt, kSh>(kmax_l, pkey, cap, a.w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                      a.w.seg_pos + (size_t)b * a.w.max_seg + wg, [&](int i) { return (uint32_t)(base + i); },
                      bkey, cap_b, a.w.cand_blk + (size_t)b * kCandCap + (size_t)wg * cap_b,
                      a.w.seg_blk + (size_t)b * a.w.max_seg + wg, [&](int i) { return (uint32_t)(base / kBlk + i); },
                      hist, red);
    } else {
      emit_segment_pair_abs<kIpt>(pkey, cap, a.w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                      a.w.seg_pos + (size_t)b * a.w.max_seg + wg, [&](int i) { return (uint32_t)(base + i); },
                      bkey, cap_b, a.w.cand_blk + (size_t)b * kCandCap + (size_t)wg * cap_b,
                      a.w.seg_blk + (size_t)b * a.w.max_seg + wg, [&](int i) { return (uint32_t)(base / kBlk + i); },
                      hist, red);
    }
  } else {
    if constexpr (kRel)
      emit_segment_m<256, kIpt, kSh>(kmax_l, pkey, cap, a.w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                                a.w.seg_pos + (size_t)b * a.w.max_seg + wg, hist, red,
                                [&](int i) { return (uint32_t)(base + i); });
    else
      emit_segment_abs<256, kIpt>(pkey, cap, a.w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                                  a.w.seg_pos + (size_t)b * a.w.max_seg + wg, hist, red,
                                  [&](int i) { return (uint32_t)(base + i); });
  }
}

// ------------------------------------------------------------------ producer: given scores
struct GivenArgs {
  const float *scores;
  int64_t stride;
  const int32_t *lens;
  int max_len;
  int K;
  SelWs w;
  uint32_t *dbg;  // debug flag word, or null
};

__global__ void __launch_bounds__(256) given_kernel(GivenArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t pkey[kScanPos];
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins];
  __shared__ uint32_t red[256 / 64 + 24];
  const int b = blockIdx.y, wg = blockIdx.x, tid = threadIdx.x;
  const int n = min(max(a.lens[b], 0), a.max_len);
  const int64_t base = (int64_t)wg * kScanPos;
  if (base >= n) return;
  zero_hists<2>(hist);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // loads first, clamped inside the row
    const int64_t p = base + 8 * tid + j;
    v[j] = a.scores[(size_t)b * a.stride + (p < n ? p : n - 1)];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) pkey[8 * tid + j] = (base + 8 * tid + j < n) ? score_key(v[j]) : 0u;
  if (a.dbg != nullptr) {
    bool fin = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) fin &= (base + 8 * tid + j >= n) || isfinite(v[j]);
    if (!fin) dbg_raise(a.dbg, kDbgScore);
  }
  __syncthreads();
  uint32_t *kout = a.w.keys + (size_t)b * a.w.cap_keys + base;
#pragma unroll
  for (int j = 0; j < 8; ++j) kout[8 * tid + j] = pkey[8 * tid + j];
  const int nseg = (n + kScanPos - 1) / kScanPos;
  const int cap = seg_budget(a.K, nseg, kScanPos);
  emit_segment<256, 8>(pkey, cap, a.w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                       a.w.seg_pos + (size_t)b * a.w.max_seg + wg, hist, red,
                       [&](int i) { return (uint32_t)(base + i); });
}

// ------------------------------------------------------------------ producer: pool scoring
struct PoolArgs {
  KvLayerDev L;
  SeqsDev S;
  const int32_t *pool;  // [B][pool_blocks]
  int pool_blocks;
  int K;
  IdxQuery q[kMaxIdxJobs];  // one query and one workspace per layer (blockIdx.z)
  SelWs w[kMaxIdxJobs];
};

// Workgroup w scores pool blocks [16w, 16w+16) of its row (wave v: blocks
// 4v .. 4v+3), stores every (key, position) and emits a budgeted segment.
template <int KF>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  constexpr bool F32 = KF == kKeyF32;
  __shared__ int64_t slot0[kPoolBlocksPerWg];
  __shared__ int32_t tok0[kPoolBlocksPerWg];
  __shared__ uint32_t key_l[256];
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins];
  __shared__ uint32_t red[256 / 64 + 24];
  const int b = blockIdx.y, wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const IdxQuery qj = a.q[blockIdx.z];
  const SelWs &w = a.w[blockIdx.z];
  const int n = row_len(a.S, b);
  if (tid < kPoolBlocksPerWg) {
    const int j = wg * kPoolBlocksPerWg + tid;
    int64_t s0 = -1;
    int t0 = -1;
    if (j < a.pool_blocks) {
      const int pb = a.pool[(size_t)b * a.pool_blocks + j];
      if (pb >= 0 && (int64_t)pb * kBlk < n) {
        const int blk = page_block(a.S, a.L.num_blocks, b, ((int64_t)pb * kBlk) / kPage);
        if (blk >= 0) {
          s0 = (int64_t)blk * kPage + ((int64_t)pb * kBlk) % kPage;
          t0 = pb * kBlk;
        }
      }
    }
    slot0[tid] = s0;
    tok0[tid] = t0;
  }
  key_l[tid] = 0u;  // items 128..255 stay empty
  zero_hists<2>(hist);
  if constexpr (KF == kKeyFp4) {
    // wave v: its 4 blocks are one tile of 32 positions (lane % 32 -> block 4 v + p / 8, position p % 8)
    Fp4Query Q;
    load_fp4_query(qj, b, a.L.idx_heads, lane, Q);
    __syncthreads();
    const int p = lane & 31, blk = 4 * wave + (p >> 3);
    const int64_t s0 = slot0[blk];
    Fp4Half kh = Fp4Half{u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, 0u};
    if (a.L.num_blocks > 0) kh = load_fp4_half(a.L, (s0 < 0 ? 0 : s0) + (p & 7), lane);  // unmapped: slot 0, masked below
    const float s = fp4_tile_score(kh, Q);
    const int t0 = tok0[blk];
    const bool ok = t0 >= 0 && t0 + (p & 7) < n;
    if (lane < 32) key_l[blk * kBlk + (p & 7)] = ok ? score_key(s) : 0u;
  } else {
  float q[8];
  {
    const float *qp = static_cast<const float *>(qj.q) + (size_t)b * kIdxDim + 8 * (lane & 7);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = qp[e];
  }
  __syncthreads();
  KeyLoad kl[4];
  if (a.L.num_blocks > 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s0 = slot0[4 * wave + u];
      kl[u] = load_unit<F32>(a.L.idx_keys, s0 < 0 ? 0 : s0, lane);  // unmapped: slot 0, masked below
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) kl[u] = KeyLoad{u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int blk = 4 * wave + u;
    const int t0 = tok0[blk];
    const float s = unit_score<F32>(kl[u], q);
    const bool ok = t0 >= 0 && t0 + (lane >> 3) < n;
    if ((lane & 7) == 0) key_l[blk * kBlk + (lane >> 3)] = ok ? score_key(s) : 0u;
  }
  }
  __syncthreads();
  auto pos_of = [&](int i) { return (uint32_t)(tok0[i >> 3] + (i & 7)); };
  if (tid < kPoolItemsPerWg) {
    const uint32_t k = key_l[tid];
    w.pool_full[(size_t)b * kMaxPoolItems + (size_t)wg * kPoolItemsPerWg + tid] =
        make_uint2(k, k ? pos_of(tid) : 0u);
  }
  const int nseg = (a.pool_blocks + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg;
  const int cap = seg_budget(a.K, nseg, kPoolItemsPerWg);
  emit_segment<256, 1>(key_l, cap, w.cand_pos + (size_t)b * kCandCap + (size_t)wg * cap,
                       w.seg_pos + (size_t)b * w.max_seg + wg, hist, red, pos_of);
}

// ------------------------------------------------------------------ select
struct SelArgs {
  SeqsDev S;
  const int32_t *lens;   // kGiven
  int max_len;           // kGiven
  int mode;
  int K;                 // indices per row
  int P;                 // pool blocks per row (kFullHier: output size; kReindex: input size)
  int32_t *pool_out;     // kFullHier
  int32_t *out[kMaxIdxJobs];  // [B][K] per job (blockIdx.z; one job except Reindex layers)
  SelWs w[kMaxIdxJobs];
};

struct SelSmem {
  uint32_t ck[kCandCap];      // candidate keys
  uint32_t cp[kCandCap];      // candidate positions
  __attribute__((aligned(16))) uint32_t hist[kBins];
  uint32_t seg_cnt[kMaxSeg];  // candidates a segment contributes
  uint32_t seg_off[kMaxSeg];  // where they start in ck/cp
  uint32_t red[80];  // scans (0..7), threshold search (16..18), per-wave values (16..23, 32..39, 48..55, 64..71), gather count (76)
  unsigned long long best;  // largest (key, ~position) of a final bin from which one item is taken
};

// Threshold of a selection: an item (key k, position p) is selected when
//   (k >> ksh) >  (kt >> ksh), or
//   (k >> ksh) == (kt >> ksh) and (!tie || ~p >= pinv).
struct Thresh {
  uint32_t kt, pinv;
  int ksh;
  bool tie;
};

// The same test as one 64-bit compare of (key, ~position) against a bound.
__device__ __forceinline__ uint64_t thresh_bound(const Thresh &th) {
  const uint32_t kf = (th.kt >> th.ksh) << th.ksh;
  return ((uint64_t)kf << 32) | (th.tie ? th.pinv : 0u);
}
__device__ __forceinline__ bool selected64(uint32_t k, uint32_t p, uint64_t bound) {
  return ((((uint64_t)k) << 32) | (uint32_t)~p) >= bound;
}
__device__ __forceinline__ bool selected(uint32_t k, uint32_t p, const Thresh &th) {
  return selected64(k, p, thresh_bound(th));
}

// Smallest key any selected item can have.
__device__ __forceinline__ uint32_t thresh_key_floor(const Thresh &th) { return (th.kt >> th.ksh) << th.ksh; }

// Exact threshold for the top `need` (1 <= need <= #valid) of n items given by
// key(i, valid) and pos(i): radix levels over the 32-bit key (digits of 11,
// 11 and 10 bits), then, only when more items than remain share the boundary
// key, over ~position among those items (lower positions win).  Each level
// builds a histogram of its digit in LDS and picks the boundary digit with
// one wave.
template <class Key, class Pos>
__device__ __forceinline__ Thresh find_thresh(SelSmem &sm, int64_t n, uint32_t need, Key key, Pos pos) {
  const int t = threadIdx.x;
  Thresh th{0u, 0u, 0, false};
  uint32_t rem = need, pre = 0, ppre = 0;
#pragma unroll 1
  for (int lv = 0; lv < 6; ++lv) {
    const bool posl = lv >= 3;
    const int l = posl ? lv - 3 : lv;
    const int sh = l == 0 ? 21 : (l == 1 ? 10 : 0);
    const int hi = l == 0 ? 32 : (l == 1 ? 21 : 10);
    const uint32_t dm = l == 2 ? 0x3FFu : 0x7FFu;
    const uint32_t hp = hi >= 32 ? 0u : ((posl ? ppre : pre) >> hi);
    for (int i = t; i < kBins; i += kSelThreads) sm.hist[i] = 0u;
    __syncthreads();
    for (int64_t i0 = t; i0 < n; i0 += 4 * kSelThreads) {
      uint32_t kk[4];
      bool vv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // reads first
        const int64_t i = i0 + u * kSelThreads;
        vv[u] = false;
        kk[u] = i < n ? key(i, vv[u]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kSelThreads;
        const uint32_t v = posl ? (vv[u] ? ~pos(i) : 0u) : kk[u];
        const bool ok = vv[u] && (!posl || kk[u] == pre) && (hi >= 32 || (v >> hi) == hp);
        if (ok) atomicAdd(&sm.hist[(v >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    find_threshold(sm.hist, rem, sm.red + 16);
    const uint32_t d = sm.red[16];
    rem -= sm.red[17];
    const bool done = sm.hist[d] == rem;
    __syncthreads();
    if (!posl) {
      pre |= d << sh;
      th.kt = pre;
      th.ksh = sh;
      if (done) return th;
      if (l == 2) th.tie = true;  // every key bit fixed: ties resolved by position
    } else {
      ppre |= d << sh;
      th.pinv = ppre & ~((1u << sh) - 1u);
      if (done) return th;
    }
  }
  return th;
}

// Ordered compaction of the selected items (or of all valid ones) of n items
// to out[0 .. out_cap); returns the count written.
template <int IPT, class Key, class Pos>
__device__ __forceinline__ uint32_t compact(SelSmem &sm, int64_t n, bool all, const Thresh &th, Key key, Pos pos,
                                            int32_t *out, uint32_t out_cap) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t written = 0;
  for (int64_t c0 = 0; c0 < n; c0 += (int64_t)kSelThreads * IPT) {
    const int64_t i0 = c0 + (int64_t)64 * IPT * wave + lane;  // this lane's items: i0 + 64 j
    uint32_t flags = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int64_t i = i0 + 64 * j;
      bool valid = false;
      uint32_t k = 0;
      if (i < n) k = key(i, valid);
      if (valid && (all || selected(k, pos(i), th))) flags |= 1u << j;
    }
    written += ordered_emit<kSelThreads, IPT>(flags, sm.red, written, [&](int j, uint32_t slot, bool keep) {
      if (keep && slot < out_cap) out[slot] = (int32_t)pos(i0 + 64 * j);  // cap: a repeated pool block
    });
  }
  return written < out_cap ? written : out_cap;
}

// The same two steps for the candidates held in LDS (ck/cp, n <= kCandCap),
// written without branches around the LDS reads: every level reads 8 items
// per thread and pass, indexes clamped inside the arrays and masked.
__device__ __forceinline__ Thresh find_thresh_lds(SelSmem &sm, int n, uint32_t need) {
  const int t = threadIdx.x;
  constexpr int kU = 8;
  Thresh th{0u, 0u, 0, false};
  uint32_t rem = need, pre = 0, ppre = 0;
#pragma unroll 1
  for (int lv = 0; lv < 6; ++lv) {
    const bool posl = lv >= 3;
    const int l = posl ? lv - 3 : lv;
    const int sh = l == 0 ? 21 : (l == 1 ? 10 : 0);
    const uint32_t hm = l == 0 ? 0u : (l == 1 ? 0xFFE00000u : 0xFFFFFC00u);  // bits fixed by earlier levels
    const uint32_t dm = l == 2 ? 0x3FFu : 0x7FFu;
    const uint32_t want = (posl ? ppre : pre) & hm;
    for (int i = t; i < kBins; i += kSelThreads) sm.hist[i] = 0u;
    __syncthreads();
    if (!posl) {
      for (int c0 = 0; c0 < n; c0 += kU * kSelThreads) {
        uint32_t k[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) k[u] = sm.ck[min(c0 + u * kSelThreads + t, kCandCap - 1)];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const bool ok = (c0 + u * kSelThreads + t < n) & (k[u] != 0u) & ((k[u] & hm) == want);
          if (ok) atomicAdd(&sm.hist[(k[u] >> sh) & dm], 1u);
        }
      }
    } else {
      for (int c0 = 0; c0 < n; c0 += kU * kSelThreads) {
        uint32_t k[kU], p[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = min(c0 + u * kSelThreads + t, kCandCap - 1);
          k[u] = sm.ck[i];
          p[u] = ~sm.cp[i];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const bool ok = (c0 + u * kSelThreads + t < n) & (k[u] != 0u) & (k[u] == pre) & ((p[u] & hm) == want);
          if (ok) atomicAdd(&sm.hist[(p[u] >> sh) & dm], 1u);
        }
      }
    }
    __syncthreads();
    find_threshold(sm.hist, rem, sm.red + 16);
    const uint32_t d = sm.red[16];
    rem -= sm.red[17];
    const bool done = sm.hist[d] == rem;
    __syncthreads();
    if (!posl) {
      pre |= d << sh;
      th.kt = pre;
      th.ksh = sh;
      if (done) return th;
      if (l == 2) th.tie = true;  // every key bit fixed: ties resolved by position
    } else {
      ppre |= d << sh;
      th.pinv = ppre & ~((1u << sh) - 1u);
      if (done) return th;
    }
  }
  return th;
}

// The candidates a select thread holds in registers: items
// i = 64 kSelIPT wave + 64 j + lane (j < kSelIPT) of the candidate array, so
// item order is (wave, j, lane) order; key 0 marks an empty item.
struct Items {
  uint32_t k[kSelIPT], p[kSelIPT];
};

__device__ __forceinline__ int item_index(int j) {
  return 64 * kSelIPT * (int)(threadIdx.x >> 6) + 64 * j + (int)(threadIdx.x & 63);
}

__device__ __forceinline__ void load_items_lds(const SelSmem &sm, int n, Items &it) {
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j) {
    const int i = item_index(j);  // < kCandCap
    it.k[j] = i < n ? sm.ck[i] : 0u;
    it.p[j] = sm.cp[i];
  }
}

// Key range [kmin, kmax] of the valid items of the workgroup (one barrier).
__device__ __forceinline__ void items_key_range(SelSmem &sm, const Items &it, uint32_t *kmin, uint32_t *kmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j) {
    hi = max(hi, it.k[j]);
    lo = min(lo, it.k[j] ? it.k[j] : 0xFFFFFFFFu);
  }
  hi = wave_inclusive_max(hi);
  lo = ~wave_inclusive_max(~lo);
  if (lane == 63) {
    sm.red[32 + wave] = hi;
    sm.red[48 + wave] = lo;
  }
  __syncthreads();
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    mx = max(mx, sm.red[32 + w]);
    mn = min(mn, sm.red[48 + w]);
  }
  *kmin = mn;
  *kmax = mx;
}

// Zeroes the histogram, the gather counter and the best-item word for find_thresh_items.
__device__ __forceinline__ void clear_for_search(SelSmem &sm) {
  u32x4 *h4 = reinterpret_cast<u32x4 *>(sm.hist), *s4 = reinterpret_cast<u32x4 *>(sm.seg_cnt);
  for (int i = threadIdx.x; i < kBins / 4; i += kSelThreads) {
    h4[i] = u32x4{0u, 0u, 0u, 0u};
    s4[i] = u32x4{0u, 0u, 0u, 0u};  // second-level histogram
  }
  if (threadIdx.x == 0) {
    sm.red[76] = 0u;
    sm.best = 0ull;
  }
}

// Exact threshold for the top `need` of the items (at least `need` valid ones;
// n = extent of the candidate array), usually in one or two histogram passes:
// digits are taken relative to the items' own key range [kmin, kmax] split
// into at most 2048 bins, so the items spread over the bins, and the
// boundary bin is split the same way once more (second-level histogram in
// seg_cnt).  At most 64 items left in the final bin are ranked by one wave
// (gathered into seg_off); more send the items to LDS for the radix levels.
// When one item of a final bin of at most 64 is taken, an LDS maximum over
// the items in place finds it instead.  On entry hist, seg_cnt[0 .. 2048), the gather
// counter red[76] and best are zero and a barrier separates the call from
// earlier reads of red[16..17], seg_off and best.
__device__ __forceinline__ Thresh find_thresh_items(SelSmem &sm, const Items &it, int n, uint32_t need,
                                                    uint32_t kmin, uint32_t kmax) {
  const int t = threadIdx.x;
  const uint32_t span = kmax - kmin;
  const int shift = span < kBins ? 0 : (32 - __clz((int)(span >> 11)));  // (span >> shift) < 2048
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j)
    if (it.k[j]) atomicAdd(&sm.hist[(it.k[j] - kmin) >> shift], 1u);
  __syncthreads();
  find_threshold(sm.hist, need, sm.red + 16);
  const uint32_t d = sm.red[16];
  uint32_t rem = need - sm.red[17];
  const uint32_t in_bin = sm.hist[d];
  Thresh th{0u, 0u, 0, false};
  if (in_bin == rem) {  // the whole boundary bin is taken
    th.kt = kmin + (d << shift);
    return th;
  }
  // second level over the boundary bin's keys [base, base + 2^shift)
  uint32_t lo_key = kmin + (d << shift);  // the items that remain are in [lo_key, lo_key + 2^sub)
  int sub = shift;
  uint32_t remaining = in_bin;
  if (shift > 0) {
    const int shift2 = shift > 11 ? shift - 11 : 0;
    uint32_t *h2 = sm.seg_cnt;
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j)
      if ((it.k[j] != 0u) & (((it.k[j] - kmin) >> shift) == d)) atomicAdd(&h2[(it.k[j] - lo_key) >> shift2], 1u);
    __syncthreads();
    find_threshold(h2, rem, sm.red + 20);
    const uint32_t d2 = sm.red[20];
    rem -= sm.red[21];
    lo_key += d2 << shift2;
    remaining = h2[d2];
    if (remaining == rem) {  // the whole second-level bin is taken
      th.kt = lo_key;
      return th;
    }
    sub = shift2;
  }
  if (remaining > 64u) {  // heavy ties or clustering: radix levels over the items in LDS
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      sm.ck[item_index(j)] = it.k[j];
      sm.cp[item_index(j)] = it.p[j];
    }
    __syncthreads();
    return find_thresh_lds(sm, n, need);
  }
  if (rem == 1u) {
    // one item of the bin (<= 64 items) is taken: the threshold item is the
    // bin's best by (key desc, position asc), one LDS maximum of
    // (key, ~position) over the items in place (no gather, no rank; a larger
    // bin of equal keys would serialize on the one word)
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j)
      if ((it.k[j] >= lo_key) & (((it.k[j] - lo_key) >> sub) == 0u))
        atomicMax(&sm.best, ((unsigned long long)it.k[j] << 32) | (unsigned long long)(~it.p[j]));
    __syncthreads();
    const unsigned long long v = sm.best;
    th.kt = (uint32_t)(v >> 32);
    th.pinv = (uint32_t)v;
    th.tie = true;
    return th;
  }
  // gather the remaining bin (<= 64 items) and rank it in wave 0
  uint32_t *gk = sm.seg_off, *gp = sm.seg_off + 64, *gn = sm.red + 76;
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j) {
    if ((it.k[j] >= lo_key) & (((it.k[j] - lo_key) >> sub) == 0u)) {
      const uint32_t slot = atomicAdd(gn, 1u);
      gk[slot] = it.k[j];
      gp[slot] = it.p[j];
    }
  }
  __syncthreads();
  if (t < 64) {
    const uint32_t cnt = *gn;
    const uint32_t mk = t < (int)cnt ? gk[t] : 0u, mp = t < (int)cnt ? gp[t] : 0xFFFFFFFFu;
    uint32_t rank = 0;  // items of the bin that come before mine: larger key, or equal key and lower position
    for (uint32_t j0 = 0; j0 < cnt; j0 += 16) {
      u32x4 kq[4], pq[4];  // 16 items per round, broadcast 16-byte reads issued together
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kq[q] = *reinterpret_cast<const u32x4 *>(gk + j0 + 4 * q);
        pq[q] = *reinterpret_cast<const u32x4 *>(gp + j0 + 4 * q);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t j = j0 + 4 * q + e, kj = kq[q][e], pj = pq[q][e];
          rank += ((j < cnt) & ((kj > mk) | ((kj == mk) & (pj < mp)))) ? 1u : 0u;
        }
    }
    // the threshold item: the last one taken (largest rank below rem)
    const bool cand = t < (int)cnt && rank < rem;
    const uint32_t r = wave_inclusive_max(cand ? rank + 1u : 0u);
    const uint32_t best = wave_last(r);
    const uint64_t who = __ballot(cand && rank + 1u == best);
    if (t == __ffsll((unsigned long long)who) - 1) {
      sm.red[16] = mk;
      sm.red[17] = ~mp;
    }
  }
  __syncthreads();
  th.kt = sm.red[16];
  th.pinv = sm.red[17];
  th.tie = true;
  return th;
}

// Ordered compaction of the selected items (all valid ones when `all`) to
// out[0 .. need), padded with -1.  Each kept position is stored from the
// register that holds it (the kept items of one ballot land in consecutive
// slots, so each store instruction writes one contiguous run; staging them in
// LDS for 16-byte stores measured slower).  Returns the number of kept items written
// (at most need).  A barrier separates the call from earlier reads of ck and
// of red[0..7].
__device__ __forceinline__ uint32_t compact_items(SelSmem &sm, const Items &it, bool all, const Thresh &th,
                                                  int32_t *out, uint32_t need) {
  constexpr int NW = kSelThreads / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint64_t bound = all ? 0ull : thresh_bound(th);
  const uint64_t below = __lanemask_lt();
  uint64_t bal[kSelIPT];
  uint32_t wtot = 0;
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j) {
    bal[j] = __ballot((it.k[j] != 0u) & selected64(it.k[j], it.p[j], bound));
    wtot += (uint32_t)__popcll(bal[j]);
  }
  if (lane == 0) sm.red[wave] = wtot;
  __syncthreads();
  uint32_t run = 0, written = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = sm.red[w];
    run += w < wave ? x : 0u;
    written += x;
  }
  // items in (wave, j, lane) order: stream order; the kept items of one
  // (wave, j) land in consecutive slots, so each store covers one run
#pragma unroll
  for (int j = 0; j < kSelIPT; ++j) {
    const uint32_t slot = run + (uint32_t)__popcll(bal[j] & below);
    if (((bal[j] >> lane) & 1u) & (slot < need)) out[slot] = (int32_t)it.p[j];  // cap: a repeated pool block
    run += (uint32_t)__popcll(bal[j]);
  }
  written = written < need ? written : need;
  for (int i = (int)written + t; i < (int)need; i += kSelThreads) out[i] = -1;
  return written;
}

// A row's candidate stream: nseg segments of ips items; segment s emitted
// info[s].count candidates at cand[s * cap ..]; every item of segment s is
// also stored: keys at full_keys[s * ips + i] (position s * ips + i) or
// (key, position) pairs at full_pairs[s * ips + i].
struct Stream {
  const uint2 *cand;
  const SegInfo *info;
  const uint32_t *full_keys;
  const uint2 *full_pairs;
  int nseg, ips, cap;
  int64_t items;  // stored items of the row (nseg * ips or fewer)
};

__device__ __forceinline__ uint2 stored_item(const Stream &s, int64_t i) {
  if (s.full_pairs) return s.full_pairs[i];
  return make_uint2(s.full_keys[i], (uint32_t)i);
}

// Exclusive prefix of v across one wave; *total gets the wave's sum.
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t v, uint32_t *total) {
  const uint32_t incl = wave_inclusive_sum(v);
  *total = wave_last(incl);
  return incl - v;
}

// One wave walks every stored item of segment s in position order and counts
// (FILL false) or writes to ck/cp from dst on (FILL true) those with a
// non-zero key >= floor_key.  Key segments hold ips = 128, 256, 1024 or 2048
// keys (one 16-byte load per lane per 256; with 128, lanes 0..31 only), pair
// segments ips = 128 pairs.
template <bool FILL>
__device__ __forceinline__ uint32_t wave_segment(SelSmem &sm, const Stream &st, int s, uint32_t floor_key, uint32_t dst) {
  const int lane = threadIdx.x & 63;
  uint32_t run = 0;
  if (st.full_pairs) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(st.full_pairs + (size_t)s * st.ips);
    const int steps = st.ips / 128;
    for (int u = 0; u < steps; ++u) {
      const u32x4 v = src[64 * u + lane];  // pairs 2*lane and 2*lane + 1 of this step
      const bool t0 = v[0] != 0u && v[0] >= floor_key, t1 = v[2] != 0u && v[2] >= floor_key;
      uint32_t tot;
      uint32_t o = run + wave_exclusive_scan((uint32_t)t0 + (uint32_t)t1, &tot);
      if constexpr (FILL) {
        if (t0) {
          sm.ck[dst + o] = v[0];
          sm.cp[dst + o] = v[1];
          ++o;
        }
        if (t1) {
          sm.ck[dst + o] = v[2];
          sm.cp[dst + o] = v[3];
        }
      }
      run += tot;
    }
  } else {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(st.full_keys + (size_t)s * st.ips);
    const int steps = (st.ips + 255) / 256;   // 1, 4 or 8
    const bool lane_ok = st.ips >= 256 || 4 * lane < st.ips;  // 128 keys: lanes 0..31
    for (int u0 = 0; u0 < steps; u0 += 4) {
    u32x4 v[4];
#pragma unroll
    for (int du = 0; du < 4; ++du)  // loads first (a masked lane reads the segment's first keys)
      v[du] = src[lane_ok ? 64 * (u0 + du < steps ? u0 + du : u0) + lane : 0];
#pragma unroll
    for (int du = 0; du < 4; ++du) {
      const int u = u0 + du;
      if (u >= steps) break;
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (lane_ok && v[du][e] != 0u && v[du][e] >= floor_key) ? 1u : 0u;
      uint32_t tot;
      uint32_t o = run + wave_exclusive_scan(c, &tot);
      if constexpr (FILL) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (lane_ok && v[du][e] != 0u && v[du][e] >= floor_key) {
            sm.ck[dst + o] = v[du][e];
            sm.cp[dst + o] = (uint32_t)((int64_t)s * st.ips + 256 * u + 4 * lane + e);
            ++o;
          }
      }
      run += tot;
    }
    }
  }
  return run;
}

// Copies every segment's emitted candidates to ck/cp at seg_off (segments in
// order, so positions stay ordered) with one load per slot: segment s owns
// slots [s * cap, s * cap + cap) of cand, of which the first seg_cnt[s] are
// filled.  When ovf_l is given, segments whose bit is set there are left out.
__device__ __forceinline__ void copy_candidates(SelSmem &sm, const Stream &st, int nseg, const uint32_t *ovf_l) {
  const int t = threadIdx.x;
  const int slots = nseg * st.cap;  // <= kCandCap
  const float inv_cap = 1.0f / (float)st.cap;
  constexpr int kBatch = 12;
#pragma unroll 1
  for (int u0 = 0; u0 < kSelIPT; u0 += kBatch) {
    if (t + kSelThreads * u0 >= slots) break;
    uint2 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = t + kSelThreads * (u0 + u);
      v[u] = st.cand[j < slots ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = t + kSelThreads * (u0 + u);
      if (j < slots) {
        int sg = (int)((float)j * inv_cap);  // j / cap, corrected below
        int i = j - sg * st.cap;
        if (i < 0) {
          --sg;
          i += st.cap;
        } else if (i >= st.cap) {
          ++sg;
          i -= st.cap;
        }
        const bool skip = ovf_l && ((ovf_l[sg >> 5] >> (sg & 31)) & 1u);
        if (!skip && (uint32_t)i < sm.seg_cnt[sg]) {
          const uint32_t d = sm.seg_off[sg] + (uint32_t)i;
          sm.ck[d] = v[u].x;
          sm.cp[d] = v[u].y;
        }
      }
    }
  }
}

// The select over every stored item of a row, for rows whose candidates do
// not fit in LDS (heavily clustered or tied scores).
__device__ __forceinline__ uint32_t select_all_stored(SelSmem &sm, const Stream &st, int need, int32_t *out) {
  const int t = threadIdx.x;
  auto gkey = [&](int64_t i, bool &valid) {
    const uint32_t k = stored_item(st, i).x;
    valid = k != 0u;
    return k;
  };
  auto gpos = [&](int64_t i) { return stored_item(st, i).y; };
  uint32_t v = 0;
  for (int64_t i = t; i < st.items; i += kSelThreads) v += stored_item(st, i).x != 0u;
  uint32_t tot;
  block_exclusive_scan<kSelThreads>(v, sm.red, &tot);
  const bool all = (int64_t)tot <= need;
  Thresh th{0u, 0u, 0, false};
  if (!all) th = find_thresh(sm, st.items, (uint32_t)need, gkey, gpos);
  return compact<2>(sm, st.items, all, th, gkey, gpos, out, (uint32_t)need);
}

// Overflow path of a selection: re-reads every segment whose edge is above
// floor_key (items at or above the floor only) next to the other segments'
// emitted candidates, into ck/cp in stream order.  Returns false when the
// selection was finished here instead (more than kCandCap items: out written
// from the stored items directly); else *n_c is the number of items in ck/cp.
__device__ __forceinline__ bool reload_overflowing(SelSmem &sm, const Stream &st, int nseg, uint32_t floor_key,
                                                   int need, int32_t *out, int *n_c) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // --- overflowing segments: a bitmap in hist (kMaxSeg bits)
  uint32_t *ovf_l = sm.hist;
  auto is_ovf = [&](int s) { return (ovf_l[s >> 5] >> (s & 31)) & 1u; };
  __syncthreads();
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kSegPerThread; ++j) {
    const int s = kSegPerThread * t + j;
    const uint32_t edge = st.info[s < nseg ? s : (nseg > 0 ? nseg - 1 : 0)].edge;
    if (s < nseg && edge > floor_key) mine |= 1u << j;
  }
  // thread t's bits land at bit kSegPerThread * (t % tpw) of word t / tpw
  {
    constexpr int tpw = 32 / kSegPerThread;
    uint32_t word = mine << (kSegPerThread * (t % tpw));
#pragma unroll
    for (int o = 1; o < tpw; o <<= 1) word |= __shfl_xor(word, o);
    if (t % tpw == 0) ovf_l[t / tpw] = word;
  }
  __syncthreads();
  // emitted counts of every segment (the overflowing ones are recounted below,
  // by other waves: the barrier orders the two writes of such a count)
#pragma unroll
  for (int j = 0; j < kSegPerThread; ++j) {
    const int s = kSegPerThread * t + j;
    if (s < nseg) sm.seg_cnt[s] = st.info[s].count;
  }
  __syncthreads();
  // --- count, one wave per overflowing segment (wave w: segments w, w+8, ...)
  for (int s = wave; s < nseg; s += kSelThreads / 64)
    if (is_ovf(s)) {
      const uint32_t c = wave_segment<false>(sm, st, s, floor_key, 0u);
      if (lane == 0) sm.seg_cnt[s] = c;
    }
  __syncthreads();
  uint32_t cnt2 = 0;
#pragma unroll
  for (int j = 0; j < kSegPerThread; ++j) {
    const int s = kSegPerThread * t + j;
    if (s < nseg) cnt2 += sm.seg_cnt[s];
  }
  uint32_t C2;
  uint32_t off2 = block_exclusive_scan<kSelThreads>(cnt2, sm.red, &C2);
  if (C2 > (uint32_t)kCandCap) {
    const uint32_t written = select_all_stored(sm, st, need, out);
    for (int i = (int)written + t; i < need; i += kSelThreads) out[i] = -1;  // slots it did not write
    return false;
  }
#pragma unroll
  for (int j = 0; j < kSegPerThread; ++j) {
    const int s = kSegPerThread * t + j;
    if (s < nseg) {
      sm.seg_off[s] = off2;
      off2 += sm.seg_cnt[s];
    }
  }
  __syncthreads();
  copy_candidates(sm, st, nseg, ovf_l);
  for (int s = wave; s < nseg; s += kSelThreads / 64)
    if (is_ovf(s)) wave_segment<true>(sm, st, s, floor_key, sm.seg_off[s]);
  __syncthreads();
  *n_c = (int)C2;
  return true;
}

// Top `need` of a row from its stream, in increasing position order (stream
// order for a pool), -1 padded.
__device__ __forceinline__ void select_stream(SelSmem &sm, const Stream &st, int need, int32_t *out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nseg = st.nseg < kMaxSeg ? st.nseg : kMaxSeg;
  const int slots = nseg * st.cap;  // <= kCandCap
  // --- every candidate slot (segment s owns slots [s cap, s cap + cap), unused
  // ones hold key 0, so slot order is position order) straight into registers,
  // and the segment infos (thread t: segments kSegPerThread t ..); all loads
  // are issued before any use
  Items it;
  {
    uint2 v[kSelIPT];
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      const int i = item_index(j);
      v[j] = st.cand[i < slots ? i : 0];
    }
    SegInfo si[kSegPerThread];
#pragma unroll
    for (int j = 0; j < kSegPerThread; ++j) {
      const int s = kSegPerThread * t + j;
      si[j] = st.info[s < nseg ? s : (nseg > 0 ? nseg - 1 : 0)];
    }
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      it.k[j] = item_index(j) < slots ? v[j].x : 0u;
      it.p[j] = v[j].y;
    }
    uint32_t cnt = 0, emax = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int j = 0; j < kSegPerThread; ++j) {
      const int s = kSegPerThread * t + j;
      if (s < nseg) emax = max(emax, si[j].edge);
    }
#pragma unroll
    for (int j = 0; j < kSelIPT; ++j) {
      hi = max(hi, it.k[j]);
      lo = min(lo, it.k[j] ? it.k[j] : 0xFFFFFFFFu);
      cnt += (uint32_t)__popcll(__ballot(it.k[j] != 0u));  // candidates: the slots with a key
    }
    // one exchange for the candidate count, the largest edge and the key range
    emax = wave_inclusive_max(emax);
    hi = wave_inclusive_max(hi);
    lo = ~wave_inclusive_max(~lo);
    if (lane == 63) {
      sm.red[16 + wave] = emax;
      sm.red[32 + wave] = hi;
      sm.red[48 + wave] = lo;
      sm.red[64 + wave] = cnt;
    }
  }
  clear_for_search(sm);
  __syncthreads();
  uint32_t max_edge = 0, kmax = 0, kmin = 0xFFFFFFFFu, C = 0;  // C: candidates in the slots
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    max_edge = max(max_edge, sm.red[16 + w]);
    kmax = max(kmax, sm.red[32 + w]);
    kmin = min(kmin, sm.red[48 + w]);
    C += sm.red[64 + w];
  }
  // (red[16..71] is next written after the histogram barrier)

  // Pass 0 selects among the emitted candidates.  Items a segment left out
  // are below its edge, so when no edge is above the selection's key floor
  // that selection is exact.  Otherwise the segments with such an edge are
  // re-read in full (items at or above the floor only) and pass 1 selects
  // among the larger set, which is then exact: its threshold can only rise.
  // (Straight-line passes: the overflow path's set-up stays off the common one.)
  int n_c = 0;
  {
    Thresh th{0u, 0u, 0, false};
    const bool all = C <= (uint32_t)need;
    if (!all) th = find_thresh_items(sm, it, slots, (uint32_t)need, kmin, kmax);
    const uint32_t floor_key = all ? 0u : thresh_key_floor(th);
    if (all ? max_edge == 0u : max_edge <= floor_key) {
      compact_items(sm, it, all, th, out, (uint32_t)need);
      return;
    }
    if (!reload_overflowing(sm, st, nseg, floor_key, need, out, &n_c)) return;
    load_items_lds(sm, n_c, it);
    clear_for_search(sm);  // the bitmap in hist was last read before reload's final barrier
    items_key_range(sm, it, &kmin, &kmax);
  }
  {
    // pass 1 over the n_c items now in LDS (all valid)
    Thresh th{0u, 0u, 0, false};
    const bool all = n_c <= need;
    if (!all) th = find_thresh_items(sm, it, n_c, (uint32_t)need, kmin, kmax);
    compact_items(sm, it, all, th, out, (uint32_t)need);
  }
}

// grid (1 or 2, B): x == 0 selects positions (indices), x == 1 the pool blocks.
__global__ void __launch_bounds__(kSelThreads) select_kernel(SelArgs a) {
  __shared__ SelSmem sm;
  const int b = blockIdx.y;
  const bool re = a.mode == kReindex, blk = blockIdx.x != 0;
  const SelWs &w = a.w[blockIdx.z];
  const int n = re ? 0 : (a.mode == kGiven ? min(max(a.lens[b], 0), a.max_len) : row_len(a.S, b));
  Stream st;
  st.cand = (blk ? w.cand_blk : w.cand_pos) + (size_t)b * kCandCap;
  st.info = (blk ? w.seg_blk : w.seg_pos) + (size_t)b * w.max_seg;
  st.full_keys = re ? nullptr : (blk ? w.bkeys + (size_t)b * w.cap_blocks : w.keys + (size_t)b * w.cap_keys);
  st.full_pairs = re ? w.pool_full + (size_t)b * kMaxPoolItems : nullptr;
  st.nseg = re ? (a.P + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg : (n + w.slice - 1) / w.slice;
  st.ips = re ? kPoolItemsPerWg : (blk ? w.slice / kBlk : w.slice);
  st.items = re ? (int64_t)a.P * kBlk : (blk ? (n + kBlk - 1) / kBlk : n);
  const int need = blk ? a.P : a.K;
  int32_t *out = blk ? a.pool_out + (size_t)b * a.P : a.out[blockIdx.z] + (size_t)b * a.K;
  st.cap = seg_budget(need, st.nseg, st.ips);
  select_stream(sm, st, need, out);
}

// ------------------------------------------------------------------ scores only
template <bool F32>
__global__ void __launch_bounds__(256) scores_kernel(KvLayerDev L, SeqsDev S, const float *q_idx, float *scores,
                                                     int units_per_wg) {
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = row_len(S, b);
  const int64_t total_units = ((int64_t)S.max_len + 7) / 8;
  const int64_t u_begin = (int64_t)blockIdx.x * units_per_wg;
  const int64_t u_end = min(u_begin + units_per_wg, total_units);
  float q[8];
  const float *qp = q_idx + (size_t)b * kIdxDim + 8 * (lane & 7);
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = qp[e];
  for (int64_t u = u_begin + wave; u < u_end; u += 4) {
    const int64_t t0 = u * 8;
    const int blk = (t0 < n && L.num_blocks > 0) ? page_block(S, L.num_blocks, b, t0 / kPage) : -1;
    KeyLoad kl = KeyLoad{u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    if (L.num_blocks > 0)  // unmapped: slot 0, masked below (an empty pool has no slot 0)
      kl = load_unit<F32>(L.idx_keys, blk < 0 ? 0 : (int64_t)blk * kPage + t0 % kPage, lane);
    const float s = unit_score<F32>(kl, q);
    const int64_t t = t0 + (lane >> 3);
    if ((lane & 7) == 0 && t < S.max_len) scores[(size_t)b * S.max_len + t] = (blk >= 0 && t < n) ? s : -INFINITY;
  }
}

// FP4 keys, multi-head score: tiles of 32 positions, a wave per tile.
__global__ void __launch_bounds__(256) scores_fp4_kernel(KvLayerDev L, SeqsDev S, IdxQuery qi, float *scores,
                                                         int tiles_per_wg) {
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = row_len(S, b);
  const int64_t total_tiles = ((int64_t)S.max_len + 31) / 32;
  const int64_t t_begin = (int64_t)blockIdx.x * tiles_per_wg;
  const int64_t t_end = min(t_begin + tiles_per_wg, total_tiles);
  Fp4Query Q;
  load_fp4_query(qi, b, L.idx_heads, lane, Q);
  for (int64_t tile = t_begin + wave; tile < t_end; tile += 4) {  // wave-uniform trip count
    const int64_t t = tile * 32 + (lane & 31);
    const int blk = (t < n && L.num_blocks > 0) ? page_block(S, L.num_blocks, b, t / kPage) : -1;
    Fp4Half kh = Fp4Half{u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, 0u};
    if (L.num_blocks > 0)  // unmapped: slot 0, masked below (an empty pool has no slot 0)
      kh = load_fp4_half(L, blk < 0 ? 0 : (int64_t)blk * kPage + t % kPage, lane);
    const float s = fp4_tile_score(kh, Q);
    if (lane < 32 && t < S.max_len) scores[(size_t)b * S.max_len + t] = (blk >= 0 && t < n) ? s : -INFINITY;
  }
}

hipError_t run_select(const SelArgs &a, int outputs, int batch, int jobs, hipStream_t st) {
  timer_before(kKernTopkCompact, st);
  select_kernel<<<dim3(outputs, batch, jobs), dim3(kSelThreads), 0, st>>>(a);
  timer_after(kKernTopkCompact, st);
  return hipGetLastError();
}

// Reindex of `jobs` layers over one pool: pool scoring and the select, each
// one launch with a grid dimension over the layers.
hipError_t run_reindex(const KvLayerDev &L, const SeqsDev &S, const IdxQuery *q, const SelWs *w,
                       int32_t *const *indices, int jobs, int top_k, const int32_t *pool_in, int pool_blocks,
                       hipStream_t st) {
  PoolArgs p{};
  p.L = L;
  p.S = S;
  p.pool = pool_in;
  p.pool_blocks = pool_blocks;
  p.K = top_k;
  for (int j = 0; j < jobs; ++j) {
    p.q[j] = q[j];
    p.w[j] = w[j];
  }
  const int gx = (pool_blocks + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg;
  const dim3 grid(gx, S.batch, jobs);
  timer_before(kKernPoolScore, st);
  if (L.idx_fp4) pool_kernel<kKeyFp4><<<grid, dim3(256), 0, st>>>(p);
  else if (L.idx_f32) pool_kernel<kKeyF32><<<grid, dim3(256), 0, st>>>(p);
  else pool_kernel<kKeyBf16><<<grid, dim3(256), 0, st>>>(p);
  timer_after(kKernPoolScore, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelArgs s{};
  for (int j = 0; j < jobs; ++j) {
    s.w[j] = w[j];
    s.out[j] = indices[j];
  }
  s.S = S;
  s.mode = kReindex;
  s.K = top_k;
  s.P = pool_blocks;
  return run_select(s, 1, S.batch, jobs, st);
}

}  // namespace

size_t topk_workspace_bytes(int batch, int max_items, int top_k) {
  (void)top_k;
  return ws_bytes_for(batch, ws_shape(batch, max_items, 0, false));
}

size_t index_select_workspace_bytes(int batch, int max_len, int top_k, int pool_blocks) {
  (void)top_k;
  return ws_bytes_for(batch, ws_shape(batch, max_len, pool_blocks, true));
}

hipError_t launch_index_scores(const KvLayerDev &L, const SeqsDev &S, IdxQuery q, float *scores, hipStream_t st) {
  if (S.batch <= 0 || S.max_len <= 0) return hipSuccess;
  if (L.idx_fp4) {
    const int64_t tiles = ((int64_t)S.max_len + 31) / 32;
    const int per = 16;
    const dim3 grid((unsigned)((tiles + per - 1) / per), (unsigned)S.batch);
    timer_before(kKernIndexScores, st);
    scores_fp4_kernel<<<grid, dim3(256), 0, st>>>(L, S, q, scores, per);
    timer_after(kKernIndexScores, st);
    return hipGetLastError();
  }
  const int64_t units = ((int64_t)S.max_len + 7) / 8;
  const int per = 64;
  const int64_t gx = (units + per - 1) / per;
  const dim3 grid((unsigned)gx, (unsigned)S.batch);
  const float *q_idx = static_cast<const float *>(q.q);
  timer_before(kKernIndexScores, st);
  if (L.idx_f32) scores_kernel<true><<<grid, dim3(256), 0, st>>>(L, S, q_idx, scores, per);
  else scores_kernel<false><<<grid, dim3(256), 0, st>>>(L, S, q_idx, scores, per);
  timer_after(kKernIndexScores, st);
  return hipGetLastError();
}

hipError_t launch_topk_scores(const float *scores, int64_t stride, const int32_t *lens, int batch, int max_len,
                              int top_k, int32_t *indices, void *ws, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  const WsShape sh = ws_shape(batch, max_len, 0, false);
  SelWs w = carve(ws, batch, sh);
  GivenArgs g{scores, stride, lens, max_len, top_k, w, debug_flags()};
  const int gx = (int)(sh.cap_keys / kScanPos);
  timer_before(kKernTopkGiven, st);
  given_kernel<<<dim3(gx, batch), dim3(256), 0, st>>>(g);
  timer_after(kKernTopkGiven, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelArgs s{};
  s.w[0] = w;
  s.lens = lens;
  s.max_len = max_len;
  s.mode = kGiven;
  s.K = top_k;
  s.out[0] = indices;
  return run_select(s, 1, batch, 1, st);
}

hipError_t launch_index_select_full(const KvLayerDev &L, const SeqsDev &S, IdxQuery q_idx, int top_k,
                                    int32_t *pool_out, int pool_blocks, int32_t *indices, void *ws,
                                    hipStream_t st, const AppendRow *app, int n_app, const void *new_key) {
  if (S.batch <= 0) return hipSuccess;
  const bool hier = pool_out != nullptr;
  const WsShape sh = ws_shape(S.batch, S.max_len, hier ? pool_blocks : 0, true);
  SelWs w = carve(ws, S.batch, sh);
  ScanArgs a{};
  a.L = L;
  a.S = S;
  a.q = q_idx;
  a.K = top_k;
  a.P = pool_blocks;
  a.w = w;
  const int gx = (int)(sh.cap_keys / sh.slice);
  a.scan_wgs = gx;
  a.n_app = n_app;
  for (int i = 0; i < n_app; ++i) a.app[i] = app[i];
  a.new_key = new_key;
  a.dbg = debug_flags();
  timer_before(kKernIndexScan, st);
  const dim3 grid(gx + n_app, S.batch);
  const bool half = sh.slice != kScanPos;
#define CSA2_SCAN(KF, H)                                                        \
  do {                                                                          \
    if (half) scan_kernel<KF, H, kScanPos / 2><<<grid, dim3(256), 0, st>>>(a);  \
    else scan_kernel<KF, H, kScanPos><<<grid, dim3(256), 0, st>>>(a);           \
  } while (0)
  if (L.idx_fp4) {
    if (hier) CSA2_SCAN(kKeyFp4, true);
    else CSA2_SCAN(kKeyFp4, false);
  } else if (L.idx_f32) {
    if (hier) CSA2_SCAN(kKeyF32, true);
    else CSA2_SCAN(kKeyF32, false);
  } else {
    if (hier) CSA2_SCAN(kKeyBf16, true);
    else CSA2_SCAN(kKeyBf16, false);
  }
#undef CSA2_SCAN
  timer_after(kKernIndexScan, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelArgs s{};
  s.w[0] = w;
  s.S = S;
  s.mode = hier ? kFullHier : kFullPos;
  s.K = top_k;
  s.P = pool_blocks;
  s.pool_out = pool_out;
  s.out[0] = indices;
  return run_select(s, hier ? 2 : 1, S.batch, 1, st);
}

hipError_t launch_index_select_reindex(const KvLayerDev &L, const SeqsDev &S, IdxQuery q_idx, int top_k,
                                       const int32_t *pool_in, int pool_blocks, int32_t *indices, void *ws,
                                       hipStream_t st) {
  if (S.batch <= 0) return hipSuccess;
  const WsShape sh = ws_shape(S.batch, S.max_len, pool_blocks, true);
  SelWs w = carve(ws, S.batch, sh);
  return run_reindex(L, S, &q_idx, &w, &indices, 1, top_k, pool_in, pool_blocks, st);
}

size_t reindex_layers_workspace_bytes(int jobs, int batch) {
  return (size_t)jobs * reindex_job_bytes(batch);
}

hipError_t launch_reindex_layers(const KvLayerDev &L, const SeqsDev &S, const IdxQuery *q_idx, int32_t *const *indices,
                                 int jobs, int top_k, const int32_t *pool_in, int pool_blocks, void *ws,
                                 hipStream_t st) {
  if (S.batch <= 0 || jobs <= 0) return hipSuccess;
  SelWs w[kMaxIdxJobs];
  for (int j = 0; j < jobs; ++j) w[j] = carve_reindex(static_cast<char *>(ws) + (size_t)j * reindex_job_bytes(S.batch), S.batch);
  return run_reindex(L, S, q_idx, w, indices, jobs, top_k, pool_in, pool_blocks, st);
}

}  // namespace csa2
