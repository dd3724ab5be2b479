// Indexer scoring, exact top-K selection and the hierarchical candidate pool.
//
// Sources: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "CSA2"
// (Full / Reindex / Reuse modes: Full and Reindex score cached indexer keys
// with their own query and select the top-K; Reuse selects nothing) and
// section "Hierarchical Sparse Indexer" (the first Full layer also gives each
// block of 8 positions the maximum score inside it and keeps the best 2048
// blocks, at most 16,384 positions, as the candidate pool that the later
// Reindex layers score).
//
// Design (ours; the pages give no kernel):
//   Stage A  streams the keys once.  A wave scores one aligned run of 8
//            positions per load (8 lanes per key, 16 B per lane, so 1 KB of
//            bf16 keys per wave instruction), turns each score into an
//            order-preserving 32-bit key, and counts the keys' top 11 bits in
//            an LDS histogram that is merged into one of 8 global replicas
//            (fewer atomics on one address).  The last workgroup of a row
//            (atomic counter, no spinning) sums the replicas and finds the
//            threshold bin T holding the K-th largest key.
//   Stage B  re-reads the 4-byte keys: keys above bin T are selected outright
//            (wave-aggregated atomic slots); keys in bin T become candidates
//            (key, position) with composite (key << 32) | ~position.  The last
//            workgroup of the row finishes with an exact radix select over
//            the candidates' remaining 53 composite bits in LDS, so equal
//            scores go to the lower position, then pads with -1.
//   Scores are fp32 dot products (fp32 or bf16 keys, fp32 query).
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int kBins = 2048;      // top 11 key bits
constexpr int kReplicas = 8;     // global histogram copies per row
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

enum ItemMode { kPos = 0, kBlockMax = 1, kPool = 2, kGiven = 3 };

struct RowState {
  uint32_t ctrA, ctrB, thr, above, nsel, ncand, total, pad;
};

struct TopkWs {
  RowState *rows;   // [B]
  uint32_t *hist;   // [B][kReplicas][kBins]
  uint32_t *keys;   // [B][cap]
  uint64_t *cand;   // [B][cap]
  int64_t cap;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

TopkWs carve(void *ws, int batch, int64_t cap) {
  char *p = static_cast<char *>(ws);
  TopkWs w;
  w.rows = reinterpret_cast<RowState *>(p);
  p += align256(sizeof(RowState) * batch);
  w.hist = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)batch * kReplicas * kBins);
  w.keys = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)batch * cap);
  w.cand = reinterpret_cast<uint64_t *>(p);
  w.cap = cap;
  return w;
}

size_t ws_bytes(int batch, int64_t cap) {
  return align256(sizeof(RowState) * batch) + align256(sizeof(uint32_t) * (size_t)batch * kReplicas * kBins) +
         align256(sizeof(uint32_t) * (size_t)batch * cap) + align256(sizeof(uint64_t) * (size_t)batch * cap);
}

// ------------------------------------------------------------------ scoring
// Lane l of a wave works on position l/8 of an aligned run of 8 and on dims
// 8*(l%8) .. 8*(l%8)+7; the 8 partial sums of a position are combined with
// three xor shuffles, so every lane ends with its position's score.
struct KeyLoad {
  uint4 a, b;  // bf16 keys use a only
};

template <bool F32>
__device__ __forceinline__ KeyLoad load_unit(const void *keys, int64_t slot0, int lane) {
  KeyLoad r;
  if constexpr (F32) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(keys) +
                                                     (slot0 + (lane >> 3)) * kIdxDim + 8 * (lane & 7));
    r.a = p[0];
    r.b = p[1];
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(keys) +
                                                     (slot0 + (lane >> 3)) * kIdxDim + 8 * (lane & 7));
    r.a = p[0];
    r.b = make_uint4(0, 0, 0, 0);
  }
  return r;
}

template <bool F32>
__device__ __forceinline__ float unit_score(const KeyLoad &k, const float (&q)[8]) {
  float s;
  if constexpr (F32) {
    s = q[0] * __uint_as_float(k.a.x);
    s = fmaf(q[1], __uint_as_float(k.a.y), s);
    s = fmaf(q[2], __uint_as_float(k.a.z), s);
    s = fmaf(q[3], __uint_as_float(k.a.w), s);
    s = fmaf(q[4], __uint_as_float(k.b.x), s);
    s = fmaf(q[5], __uint_as_float(k.b.y), s);
    s = fmaf(q[6], __uint_as_float(k.b.z), s);
    s = fmaf(q[7], __uint_as_float(k.b.w), s);
  } else {
    s = q[0] * __uint_as_float(k.a.x << 16);
    s = fmaf(q[1], __uint_as_float(k.a.x & 0xFFFF0000u), s);
    s = fmaf(q[2], __uint_as_float(k.a.y << 16), s);
    s = fmaf(q[3], __uint_as_float(k.a.y & 0xFFFF0000u), s);
    s = fmaf(q[4], __uint_as_float(k.a.z << 16), s);
    s = fmaf(q[5], __uint_as_float(k.a.z & 0xFFFF0000u), s);
    s = fmaf(q[6], __uint_as_float(k.a.w << 16), s);
    s = fmaf(q[7], __uint_as_float(k.a.w & 0xFFFF0000u), s);
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  return s;
}

// Physical slot of position t0 (a multiple of 8) of row b, or -1 when its
// page is not mapped.
__device__ __forceinline__ int64_t slot_of(const SeqsDev &S, int num_blocks, int b, int64_t t0) {
  const int64_t page = t0 / kPage;
  if (page >= S.max_blocks) return -1;
  const int blk = S.block_table[(int64_t)b * S.max_blocks + page];
  if (blk < 0 || blk >= num_blocks) return -1;
  return (int64_t)blk * kPage + (t0 % kPage);
}

__device__ __forceinline__ int row_len(const SeqsDev &S, int b) {
  const int n = S.seq_lens[b];
  return n < 0 ? 0 : (n > S.max_len ? S.max_len : n);
}

// ------------------------------------------------------------------ scans
// hist: kBins counts in LDS.  Finds the bin d with
//   sum(hist[d+1..]) < need <= sum(hist[d..])
// and returns d and sum(hist[d+1..]).  When all bins together hold fewer than
// `need`, returns d = 0 and sum(hist[1..]).  Called by all kThreads threads;
// red is LDS scratch of 2 * kThreads + 4 words.
__device__ void find_threshold_bin(const uint32_t *hist, uint32_t need, uint32_t *red, uint32_t &bin,
                                   uint32_t &above) {
  const int t = threadIdx.x;
  constexpr int per = kBins / kThreads;  // thread t owns bins [per*t, per*t + per)
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) mine += hist[per * t + j];
  red[t] = mine;
  __syncthreads();
  if (t < 64) {
    uint32_t v[4];
    uint32_t lane_sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = red[4 * t + j];
      lane_sum += v[j];
    }
    uint32_t incl = lane_sum;  // inclusive suffix sum over lanes t..63
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(incl, off);
      if (t + off < 64) incl += o;
    }
    uint32_t run = incl - lane_sum;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      red[kThreads + 4 * t + j] = run;  // sum of the threads above thread 4t+j
      run += v[j];
    }
    if (t == 0) {
      red[2 * kThreads] = 0u;
      red[2 * kThreads + 1] = 0xFFFFFFFFu;
      red[2 * kThreads + 2] = incl;  // total
    }
  }
  __syncthreads();
  uint32_t run = red[kThreads + t];
#pragma unroll
  for (int j = per - 1; j >= 0; --j) {
    const uint32_t h = hist[per * t + j];
    if (run < need && run + h >= need) {
      red[2 * kThreads] = (uint32_t)(per * t + j);
      red[2 * kThreads + 1] = run;
    }
    run += h;
  }
  __syncthreads();
  bin = red[2 * kThreads];
  above = red[2 * kThreads + 1];
  if (above == 0xFFFFFFFFu) {
    bin = 0;
    above = red[2 * kThreads + 2] - hist[0];
  }
  __syncthreads();
}

// ------------------------------------------------------------------ stage A
struct StageA {
  KvLayerDev L;
  SeqsDev S;
  const float *q_idx;     // [B][64]
  const int32_t *pool;    // kPool: [B][pool_blocks]
  int pool_blocks;
  const float *scores;    // kGiven: [B][stride]
  int64_t stride;
  const int32_t *lens;    // kGiven: [B]
  int units_per_wg;       // units of 8 items (kBlockMax: 8 positions -> 1 item)
  uint32_t need;
  TopkWs w;
};

__device__ __forceinline__ void hist_add(uint32_t *h, uint32_t key) {
  if (key != 0u) atomicAdd(&h[key >> 21], 1u);
}

// After the workgroup's keys and histogram are in memory: count the
// workgroup done; the last one of the row sums the replicas (reading and
// zeroing them with atomic exchanges) and stores the threshold bin.
__device__ void stage_a_finish(const StageA &a, int b, uint32_t *sh_hist, uint32_t *red) {
  __shared__ uint32_t is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&a.w.rows[b].ctrA, 1u);
    is_last = (old == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  uint32_t *g = a.w.hist + (size_t)b * kReplicas * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) {
    uint32_t s = 0;
#pragma unroll
    for (int r = 0; r < kReplicas; ++r) s += atomicExch(&g[r * kBins + i], 0u);
    sh_hist[i] = s;
  }
  __syncthreads();
  uint32_t bin, above;
  find_threshold_bin(sh_hist, a.need, red, bin, above);
  if (threadIdx.x == 0) {
    RowState &rs = a.w.rows[b];
    rs.thr = bin;
    rs.above = above;
    rs.total = red[2 * kThreads + 2];
    rs.ctrA = 0u;
  }
}

template <int MODE, bool F32>
__global__ void __launch_bounds__(kThreads) stage_a_kernel(StageA a) {
  __shared__ uint32_t sh_hist[kBins];
  __shared__ uint32_t red[2 * kThreads + 4];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kBins; i += kThreads) sh_hist[i] = 0u;
  __syncthreads();

  uint32_t *keys_out = a.w.keys + (size_t)b * a.w.cap;
  const int64_t u_begin = (int64_t)blockIdx.x * a.units_per_wg;

  if constexpr (MODE == kGiven) {
    const int64_t n = a.lens[b] < 0 ? 0 : min((int64_t)a.lens[b], a.w.cap);
    const int64_t i_begin = u_begin * 8, i_end = i_begin + (int64_t)a.units_per_wg * 8;
    for (int64_t i = i_begin + tid; i < i_end && i < n; i += kThreads) {
      const uint32_t key = score_key(a.scores[(size_t)b * a.stride + i]);
      keys_out[i] = key;
      hist_add(sh_hist, key);
    }
  } else {
    const int n = row_len(a.S, b);
    int64_t n_units;  // units of this row
    if constexpr (MODE == kPool) n_units = a.pool_blocks;
    else n_units = (n + 7) / 8;
    const int64_t u_end = min(u_begin + a.units_per_wg, n_units);
    float q[8];
    {
      const float *qp = a.q_idx + (size_t)b * kIdxDim + 8 * (lane & 7);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = qp[e];
    }
    constexpr int kUnroll = 4;
    for (int64_t u0 = u_begin + wave; u0 < u_end; u0 += kWaves * kUnroll) {
      KeyLoad kl[kUnroll];
      int64_t t0[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t u = u0 + (int64_t)j * kWaves;
        ok[j] = false;
        t0[j] = -1;
        if (u < u_end) {
          if constexpr (MODE == kPool) {
            const int pb = a.pool[(size_t)b * a.pool_blocks + u];
            t0[j] = pb < 0 ? -1 : (int64_t)pb * 8;
          } else {
            t0[j] = u * 8;
          }
          if (t0[j] >= 0 && t0[j] < n) {
            const int64_t slot0 = slot_of(a.S, a.L.num_blocks, b, t0[j]);
            if (slot0 >= 0) {
              ok[j] = true;
              kl[j] = load_unit<F32>(a.L.idx_keys, slot0, lane);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t u = u0 + (int64_t)j * kWaves;
        if (u >= u_end) continue;  // uniform across the wave
        float s = 0.0f;
        if (ok[j]) s = unit_score<F32>(kl[j], q);
        const bool pos_ok = ok[j] && (t0[j] + (lane >> 3) < n);
        if constexpr (MODE == kBlockMax) {
          float m = pos_ok ? s : -INFINITY;
          m = fmaxf(m, __shfl_xor(m, 8));
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          if (lane == 0) {
            const uint32_t key = ok[j] ? score_key(m) : 0u;
            keys_out[u] = key;
            hist_add(sh_hist, key);
          }
        } else {
          // items of a row: positions < n (kPos) or all pool_blocks * 8 slots (kPool)
          const bool in_row = MODE == kPool || u * 8 + (lane >> 3) < n;
          if ((lane & 7) == 0 && in_row) {
            const uint32_t key = pos_ok ? score_key(s) : 0u;
            keys_out[u * 8 + (lane >> 3)] = key;
            hist_add(sh_hist, key);
          }
        }
      }
    }
  }
  __syncthreads();
  // merge the workgroup histogram into replica blockIdx.x % kReplicas
  uint32_t *g = a.w.hist + ((size_t)b * kReplicas + (blockIdx.x % kReplicas)) * kBins;
  for (int i = tid; i < kBins; i += kThreads) {
    const uint32_t c = sh_hist[i];
    if (c) atomicAdd(&g[i], c);
  }
  stage_a_finish(a, b, sh_hist, red);
}

// ------------------------------------------------------------------ stage B
struct StageB {
  SeqsDev S;
  int mode;               // ItemMode
  const int32_t *pool;    // kPool
  int pool_blocks;
  const int32_t *lens;    // kGiven
  int items_per_wg;
  uint32_t need;
  int32_t *out;           // [B][need]
  TopkWs w;
};

__device__ __forceinline__ int64_t items_of_row(const StageB &a, int b) {
  if (a.mode == kGiven) return a.lens[b] < 0 ? 0 : min((int64_t)a.lens[b], a.w.cap);
  const int n = row_len(a.S, b);
  if (a.mode == kPos) return n;
  if (a.mode == kBlockMax) return (n + 7) / 8;
  return (int64_t)a.pool_blocks * 8;
}

__device__ __forceinline__ int32_t position_of(const StageB &a, int b, int64_t i) {
  if (a.mode == kPool) return a.pool[(size_t)b * a.pool_blocks + (i >> 3)] * 8 + (int32_t)(i & 7);
  return (int32_t)i;
}

// Wave-aggregated append: every lane with `pred` gets a distinct slot.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t *counter) {
  const uint64_t m = __ballot(pred);
  const uint32_t cnt = (uint32_t)__popcll(m);
  const int lane = threadIdx.x & 63;
  const int leader = m ? __ffsll((unsigned long long)m) - 1 : 0;
  uint32_t base = 0;
  if (cnt && lane == leader) base = atomicAdd(counter, cnt);
  base = __shfl(base, leader);
  const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
  return base + (uint32_t)__popcll(below);
}

__global__ void __launch_bounds__(kThreads) stage_b_kernel(StageB a) {
  __shared__ uint32_t sh_hist[kBins];
  __shared__ uint32_t red[2 * kThreads + 4];
  __shared__ uint32_t is_last, emitted;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  RowState &rs = a.w.rows[b];
  const uint32_t thr = rs.thr;
  const int64_t items = items_of_row(a, b);
  const uint32_t *keys = a.w.keys + (size_t)b * a.w.cap;
  uint64_t *cand = a.w.cand + (size_t)b * a.w.cap;
  int32_t *out = a.out + (size_t)b * a.need;

  const int64_t i_begin = (int64_t)blockIdx.x * a.items_per_wg;
  const int64_t i_end = i_begin + a.items_per_wg;
  for (int64_t i0 = i_begin; i0 < i_end; i0 += kThreads) {
    const int64_t i = i0 + tid;
    const uint32_t key = (i < items && i < i_end) ? keys[i] : 0u;
    const uint32_t bin = key >> 21;
    const bool sure = key != 0u && bin > thr;
    const bool maybe = key != 0u && bin == thr;
    const uint32_t s_slot = wave_append(sure, &rs.nsel);
    if (sure) out[s_slot] = position_of(a, b, i);
    const uint32_t c_slot = wave_append(maybe, &rs.ncand);
    if (maybe) cand[c_slot] = ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)position_of(a, b, i));
  }

  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&rs.ctrB, 1u);
    is_last = (old == gridDim.x - 1) ? 1u : 0u;
    emitted = 0u;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  const uint32_t above = rs.above;
  const uint32_t nc = rs.ncand;
  const uint32_t total = rs.total;
  const uint32_t take = (total < a.need ? total : a.need) - above;  // candidates to keep
  auto emit = [&](uint64_t c) {
    const uint32_t slot = above + atomicAdd(&emitted, 1u);
    out[slot] = (int32_t)(~(uint32_t)(c & 0xFFFFFFFFull));
  };
  if (take >= nc) {
    for (uint32_t i = tid; i < nc; i += kThreads) emit(cand[i]);
  } else {
    uint64_t prefix = (uint64_t)thr << 53;
    uint64_t mask = 0x7FFull << 53;
    uint32_t need = take;
    const int shifts[5] = {42, 32, 21, 10, 0};
    const int widths[5] = {11, 10, 11, 11, 10};
    for (int lv = 0; lv < 5; ++lv) {
      const int sh = shifts[lv];
      const uint64_t dm = (1ull << widths[lv]) - 1ull;
      for (int i = tid; i < kBins; i += kThreads) sh_hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < nc; i += kThreads) {
        const uint64_t c = cand[i];
        if ((c & mask) == prefix) atomicAdd(&sh_hist[(c >> sh) & dm], 1u);
      }
      __syncthreads();
      uint32_t d, above_d;
      find_threshold_bin(sh_hist, need, red, d, above_d);
      for (uint32_t i = tid; i < nc; i += kThreads) {
        const uint64_t c = cand[i];
        if ((c & mask) == prefix && ((c >> sh) & dm) > d) emit(c);
      }
      need -= above_d;
      prefix |= (uint64_t)d << sh;
      mask |= dm << sh;
      const uint32_t at_d = sh_hist[d];
      __syncthreads();
      if (at_d == need) {
        for (uint32_t i = tid; i < nc; i += kThreads) {
          const uint64_t c = cand[i];
          if ((c & mask) == prefix) emit(c);
        }
        break;
      }
    }
  }
  __syncthreads();
  const uint32_t filled = above + emitted;
  for (uint32_t i = filled + tid; i < a.need; i += kThreads) out[i] = -1;
  __syncthreads();
  if (tid == 0) {
    rs.ctrB = 0u;
    rs.thr = 0u;
    rs.above = 0u;
    rs.nsel = 0u;
    rs.ncand = 0u;
    rs.total = 0u;
  }
}

// ------------------------------------------------------------------ scores only
template <bool F32>
__global__ void __launch_bounds__(kThreads) scores_kernel(KvLayerDev L, SeqsDev S, const float *q_idx, float *scores,
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
  for (int64_t u = u_begin + wave; u < u_end; u += kWaves) {
    const int64_t t0 = u * 8;
    bool ok = false;
    KeyLoad kl;
    if (t0 < n) {
      const int64_t slot0 = slot_of(S, L.num_blocks, b, t0);
      if (slot0 >= 0) {
        ok = true;
        kl = load_unit<F32>(L.idx_keys, slot0, lane);
      }
    }
    float s = ok ? unit_score<F32>(kl, q) : 0.0f;
    const int64_t t = t0 + (lane >> 3);
    if ((lane & 7) == 0 && t < S.max_len) scores[(size_t)b * S.max_len + t] = (ok && t < n) ? s : -INFINITY;
  }
}

template <int MODE>
hipError_t run_stage_a(const StageA &a, int64_t units_per_row, int batch, hipStream_t st) {
  const int64_t gx = (units_per_row + a.units_per_wg - 1) / a.units_per_wg;
  if (gx <= 0 || batch <= 0) return hipSuccess;
  const dim3 grid((unsigned)gx, (unsigned)batch);
  if (a.L.idx_f32) stage_a_kernel<MODE, true><<<grid, dim3(kThreads), 0, st>>>(a);
  else stage_a_kernel<MODE, false><<<grid, dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t run_stage_b(const StageB &a, int64_t items_per_row, int batch, hipStream_t st) {
  const int64_t gx = (items_per_row + a.items_per_wg - 1) / a.items_per_wg;
  if (gx <= 0 || batch <= 0) return hipSuccess;
  stage_b_kernel<<<dim3((unsigned)gx, (unsigned)batch), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

constexpr int kPosUnitsPerWg = 128;   // 1024 positions per workgroup in a full scan
constexpr int kPoolUnitsPerWg = 16;   // 16 pool blocks (128 positions) per workgroup
constexpr int kItemsPerWgB = 2048;    // stage B items per workgroup

}  // namespace

size_t topk_workspace_bytes(int batch, int max_items, int top_k) {
  (void)top_k;
  return ws_bytes(batch, max_items > 0 ? max_items : 1);
}

size_t index_select_workspace_bytes(int batch, int max_len, int top_k, int pool_blocks) {
  (void)top_k;
  int64_t cap = max_len;
  if ((int64_t)pool_blocks * 8 > cap) cap = (int64_t)pool_blocks * 8;
  return ws_bytes(batch, cap > 0 ? cap : 1);
}

hipError_t launch_index_scores(const KvLayerDev &L, const SeqsDev &S, const float *q_idx, float *scores,
                               hipStream_t st) {
  const int64_t units = ((int64_t)S.max_len + 7) / 8;
  const int per = 64;
  const int64_t gx = (units + per - 1) / per;
  if (gx <= 0 || S.batch <= 0) return hipSuccess;
  const dim3 grid((unsigned)gx, (unsigned)S.batch);
  if (L.idx_f32) scores_kernel<true><<<grid, dim3(kThreads), 0, st>>>(L, S, q_idx, scores, per);
  else scores_kernel<false><<<grid, dim3(kThreads), 0, st>>>(L, S, q_idx, scores, per);
  return hipGetLastError();
}

hipError_t launch_topk_scores(const float *scores, int64_t stride, const int32_t *lens, int batch, int max_len,
                              int top_k, int32_t *indices, void *ws, hipStream_t st) {
  TopkWs w = carve(ws, batch, max_len > 0 ? max_len : 1);
  StageA a{};
  a.scores = scores;
  a.stride = stride;
  a.lens = lens;
  a.units_per_wg = 256;  // 2048 scores per workgroup
  a.need = (uint32_t)top_k;
  a.w = w;
  hipError_t e = run_stage_a<kGiven>(a, ((int64_t)max_len + 7) / 8, batch, st);
  if (e != hipSuccess) return e;
  StageB bb{};
  bb.mode = kGiven;
  bb.lens = lens;
  bb.items_per_wg = kItemsPerWgB;
  bb.need = (uint32_t)top_k;
  bb.out = indices;
  bb.w = w;
  return run_stage_b(bb, max_len, batch, st);
}

hipError_t launch_index_select_full(const KvLayerDev &L, const SeqsDev &S, const float *q_idx, int top_k,
                                    int32_t *pool_out, int pool_blocks, int32_t *indices, void *ws,
                                    hipStream_t st) {
  int64_t cap = S.max_len;
  if ((int64_t)pool_blocks * 8 > cap) cap = (int64_t)pool_blocks * 8;
  TopkWs w = carve(ws, S.batch, cap > 0 ? cap : 1);
  const int64_t units = ((int64_t)S.max_len + 7) / 8;
  hipError_t e;
  if (pool_out == nullptr) {
    StageA a{};
    a.L = L; a.S = S; a.q_idx = q_idx; a.units_per_wg = kPosUnitsPerWg; a.need = (uint32_t)top_k; a.w = w;
    if ((e = run_stage_a<kPos>(a, units, S.batch, st)) != hipSuccess) return e;
    StageB bb{};
    bb.S = S; bb.mode = kPos; bb.items_per_wg = kItemsPerWgB; bb.need = (uint32_t)top_k; bb.out = indices; bb.w = w;
    return run_stage_b(bb, S.max_len, S.batch, st);
  }
  // hierarchical: block maxima -> pool blocks -> this layer's top-K inside the pool
  StageA a{};
  a.L = L; a.S = S; a.q_idx = q_idx; a.units_per_wg = kPosUnitsPerWg; a.need = (uint32_t)pool_blocks; a.w = w;
  if ((e = run_stage_a<kBlockMax>(a, units, S.batch, st)) != hipSuccess) return e;
  StageB bb{};
  bb.S = S; bb.mode = kBlockMax; bb.items_per_wg = kItemsPerWgB; bb.need = (uint32_t)pool_blocks; bb.out = pool_out;
  bb.w = w;
  if ((e = run_stage_b(bb, units, S.batch, st)) != hipSuccess) return e;
  return launch_index_select_reindex(L, S, q_idx, top_k, pool_out, pool_blocks, indices, ws, st);
}

hipError_t launch_index_select_reindex(const KvLayerDev &L, const SeqsDev &S, const float *q_idx, int top_k,
                                       const int32_t *pool_in, int pool_blocks, int32_t *indices, void *ws,
                                       hipStream_t st) {
  int64_t cap = S.max_len;
  if ((int64_t)pool_blocks * 8 > cap) cap = (int64_t)pool_blocks * 8;
  TopkWs w = carve(ws, S.batch, cap > 0 ? cap : 1);
  StageA a{};
  a.L = L; a.S = S; a.q_idx = q_idx; a.pool = pool_in; a.pool_blocks = pool_blocks;
  a.units_per_wg = kPoolUnitsPerWg; a.need = (uint32_t)top_k; a.w = w;
  hipError_t e = run_stage_a<kPool>(a, pool_blocks, S.batch, st);
  if (e != hipSuccess) return e;
  StageB bb{};
  bb.S = S; bb.mode = kPool; bb.pool = pool_in; bb.pool_blocks = pool_blocks; bb.items_per_wg = kItemsPerWgB;
  bb.need = (uint32_t)top_k; bb.out = indices; bb.w = w;
  return run_stage_b(bb, (int64_t)pool_blocks * 8, S.batch, st);
}

}  // namespace csa2
