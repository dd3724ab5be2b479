// CED global-KV projection with the FP4 pack fused into the epilogue.
//
// Source: discuss.pytorch.kr DeepSeek-V4.1-Flash summary, section "Causal
// Encoder-Decoder": every decoder layer l takes its global KV from the last
// encoder hidden state through its own weights, C_l = H W_l^KV and
// Z_l = H W_l^Z.  The FP4 format of C is the one in section "FP4 KV cache".
//
// Design (ours): all layers form one GEMM
//   out[t][n] = sum_k H[t][k] * W[n][k],  n = l * 576 + c  (c < 512: C_l, else Z_l),
//   or n = l * 512 + c when no W^Z is given
// with H [tokens][hidden] and the weights in out x in orientation, so both
// operands are read along k (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
// A workgroup of 8 waves computes a 256 x 256 output tile (128 x 64 per wave,
// 4 x 2 MFMA tiles of 32 x 32).  The tiles of each 32-wide k-step travel from
// global memory straight into LDS (global_load_lds_dwordx4, no register
// staging) three k-steps ahead of the one being multiplied, through four 32 KB
// stages; one barrier per k-step, and the outstanding loads are waited for
// per wave with an explicit vector-memory count instead of a fenced barrier.
// The tiles are dealt so that each XCD's L2 serves a block of neighbouring
// tiles.  The epilogue parks the fp32 tile in LDS 64 rows at a time and packs
// each 16-channel group of C straight to E2M1 + E4M3 (the same rounding rules
// as the standalone pack) and rounds Z to bf16, so C never reaches HBM in fp32
// (unless the optional debug copy is asked for).
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int BM = 256, BK = 32;             // workgroup tile rows, k-step
constexpr int kWM = 128, kWN = 64;           // wave tile: 4 x 2 MFMA tiles of 32 x 32
constexpr int kGroupM = 8;                   // row tiles an XCD sweeps across the columns together
constexpr int kXcds = 8;
// output columns per layer: 512 of C, then 64 of Z when W^Z is given
__device__ __forceinline__ int per_layer(const void *w_z) { return w_z != nullptr ? kLatent + kIdxDim : kLatent; }

struct CedArgs {
  const uint16_t *h;
  const uint16_t *w_kv;
  const uint16_t *w_z;
  int64_t tokens;
  int hidden;
  int n_layers;
  uint8_t *codes;
  uint8_t *scales;
  uint16_t *z;
  float *c_f32;
};

// Row n (< the total column count) of the combined weight matrix.
__device__ __forceinline__ const uint16_t *weight_row(const CedArgs &a, int n) {
  const int npl = per_layer(a.w_z);
  const int l = n / npl, c = n % npl;
  if (c < kLatent) return a.w_kv + ((size_t)l * kLatent + c) * a.hidden;
  return a.w_z + ((size_t)l * kIdxDim + (c - kLatent)) * a.hidden;
}

// One k-step stage: rows 0..255 hold the A tile (tokens), 256..511 the B tile
// (output columns), 32 bf16 of k each (64 bytes = four 16-byte chunks).  The
// chunks of a row are stored in a row-dependent order (chunk c at position
// c ^ swz(row)), so that the 16 lanes of one phase of a fragment read (16
// consecutive rows, one logical chunk) hit 16 different 16-byte bank groups
// with 64 banks, and 8 lanes hit 8 with 32.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// LDS of a workgroup with BN output columns, NST stages and an epilogue of
// RE rows at a time.
template <int BN, int NST, int RE>
union SmemCed {
  uint16_t st[NST][BM + BN][BK];  // (256 + BN) x 64 bytes per stage
  float c[RE][BN + 4];            // one epilogue round
};

// Pack (C) or round (Z) the 16 consecutive outputs v of token t, column n.
__device__ __forceinline__ void store_group(const CedArgs &a, int64_t t, int n, const float (&v)[16]) {
  const int l = n / per_layer(a.w_z), c = n % per_layer(a.w_z);
  const size_t row = (size_t)l * a.tokens + t;
  if (c < kLatent) {
    if (a.codes != nullptr) {  // null: the caller finishes C (norm, rotation) before packing
      uint32_t w0, w1;
      const uint32_t sc = pack_group16(v, &w0, &w1);
      reinterpret_cast<uint2 *>(a.codes + row * (kLatent / 2))[c / kGroup] = make_uint2(w0, w1);
      a.scales[row * (kLatent / kGroup) + c / kGroup] = (uint8_t)sc;
    }
    if (a.c_f32 != nullptr) {
      float4 *dst = reinterpret_cast<float4 *>(a.c_f32 + row * kLatent + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  } else if (a.z != nullptr) {
    uint32_t packed[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo = __float_as_uint(v[2 * i]), hi = __float_as_uint(v[2 * i + 1]);
      lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
      hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
      packed[i] = lo | (hi << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(a.z + row * kIdxDim + (c - kLatent));
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  }
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: expcnt and
// lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Workgroup barrier that orders the LDS accesses around it (the compiler may
// not move memory operations across it) without waiting for outstanding
// global-to-LDS loads the way a fenced barrier would.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// 256 x 256 output tile per workgroup, 8 waves of 128 x 64 (8 independent
// 32 x 32 accumulators per wave: each A fragment feeds 2 MFMAs, each B
// fragment 4).  The tiles travel from global memory straight into LDS
// (global_load_lds_dwordx4: 16 bytes per lane, a wave's 64 lanes fill 1 KB =
// 16 rows of a stage), three k-steps ahead of the one being multiplied.
template <int BN, int NST>
__global__ void __launch_bounds__(2 * BN) ced_kernel(CedArgs a) {
  constexpr int kWavesN = BN / kWN;             // waves across the columns (2 rows of waves)
  constexpr int kThreads = 64 * 2 * kWavesN;    // 8 waves (BN 256) or 4 (BN 128)
  constexpr int kGroups = (BM + BN) / 16 / (2 * kWavesN);  // 16-row groups a wave loads per stage
  constexpr int kRowsEpi = NST * (BM + BN) * BK * 2 >= 128 * (BN + 4) * 4 ? 128 : 64;
  __shared__ __attribute__((aligned(16))) SmemCed<BN, NST, kRowsEpi> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Tile order: the hardware deals workgroups to the 8 XCDs round-robin by
  // linear id, so the id is first renumbered to give each XCD a contiguous
  // range of tiles, which is then walked kGroupM row tiles at a time across
  // the columns: the workgroups an XCD runs together share A row tiles and B
  // column tiles in its L2.  (A bijection on the tiles; without a multiple of
  // 8 tiles the XCD step is left out.)
  const int nt = gridDim.x, mt = gridDim.y, total = nt * mt;
  const int pid = blockIdx.y * nt + blockIdx.x;
  const int t = total % kXcds == 0 ? (pid % kXcds) * (total / kXcds) + pid / kXcds : pid;
  const int first_m = (t / (kGroupM * nt)) * kGroupM;
  const int gm = min(mt - first_m, kGroupM);
  const int u = t % (kGroupM * nt);
  const int64_t m0 = (int64_t)(first_m + u % gm) * BM;
  const int n0 = (u / gm) * BN;
  const int n_total = a.n_layers * per_layer(a.w_z);
  const int wm = (wave / kWavesN) * kWM, wn = (wave % kWavesN) * kWN;

  // ---- loads: the row groups of 16 rows of a stage (16 of A, BN / 16 of B),
  // kGroups per wave; lane i fetches row 16 g + i / 4, stored chunk i % 4 =
  // logical chunk (i % 4) ^ swz
  const uint16_t *src[kGroups];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const int g = kGroups * wave + q;   // row group (0..15: A, then B)
    const int r = 16 * (g < 16 ? g : g - 16) + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(r);
    if (g < 16) {
      const int64_t m = min(m0 + r, a.tokens - 1);  // rows past the end are read from the last one, not stored
      src[q] = a.h + m * a.hidden + 8 * chunk;
    } else {
      const int n = min(n0 + r, n_total - 1);
      src[q] = weight_row(a, n) + 8 * chunk;
    }
  }
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int g = kGroups * wave + q;
      __builtin_amdgcn_global_load_lds((glb_void *)(src[q] + k0), (lds_void *)&sm.st[stage][16 * g][0], 16, 0, 0);
    }
  };

  // fragment reads: lane l takes row (l % 32) of a 32-row tile and logical
  // chunk 2 kk + l / 32 of k-step half kk, stored at chunk ^ swz(row), and
  // swz(row) depends only on l % 16 here
  const int fsw = swz(lane & 15);
  auto frags = [&](int stage, int kk, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
    const int ch = (2 * kk + (lane >> 5)) ^ fsw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[i] = *reinterpret_cast<const bf16x8 *>(&sm.st[stage][wm + 32 * i + (lane & 31)][8 * ch]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = *reinterpret_cast<const bf16x8 *>(&sm.st[stage][BM + wn + 32 * j + (lane & 31)][8 * ch]);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // ---- pipeline (k_steps = hidden / 32 >= 2).  Stage s lives in buffer
  // s % NST.  Iteration s: read the second half of stage s, multiply the
  // first; wait for this wave's loads of stage s + 1 and pass a barrier (then
  // every wave's stage s + 1 has landed and every wave is done with stage
  // s - 1); start the loads of stage s + NST - 1 into stage s - 1's buffer;
  // read the first half of stage s + 1; multiply the second half of stage s.
  // NST - 1 stages are loaded ahead (NST = 3 to 5), so a load has NST - 2
  // iterations to land.
  const int k_steps = a.hidden / BK;
  constexpr int kAhead = NST - 1;  // stages loaded ahead of the one being multiplied
  static_assert(NST >= 3 && NST <= 5, "3 to 5 stages");
  // wait until at most n stages of this wave's loads are still in flight
  auto wait_stages = [&](int n) {
    if (n <= 0) wait_vm<0>();
    else if (n == 1) wait_vm<kGroups>();
    else if (n == 2) wait_vm<2 * kGroups>();
    else wait_vm<3 * kGroups>();
  };
  const int pro = min(kAhead, k_steps);  // stages loaded up front
#pragma unroll
  for (int p = 0; p < kAhead; ++p)
    if (p < pro) issue(p, p * BK);
  wait_stages(pro - 1);  // stage 0 has landed
  barrier_lds();
  bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
  frags(0, 0, fa0, fb0);
  int s = 0;
  // steady state: no conditions in the body, so the fragment reads of the
  // next stage stay in flight while the second half's MFMAs wait only for
  // their own reads
  for (; s + kAhead < k_steps; ++s) {
    frags(s % NST, 1, fa1, fb1);
    mfmas(fa0, fb0);
    // schedule: the second half's 6 fragment reads go out between the first
    // MFMAs, so they land while the rest of the first half runs
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
    wait_vm<(kAhead - 2) * kGroups>();  // stages s + 2 .. s + kAhead - 1 may still be in flight
    barrier_lds();
    issue((s + kAhead) % NST, (s + kAhead) * BK);
    frags((s + 1) % NST, 0, fa0, fb0);
    mfmas(fa1, fb1);
    // schedule: the loads and the next stage's 6 fragment reads between the
    // second half's MFMAs
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
  for (; s < k_steps; ++s) {  // the last stages: everything is loaded or in flight
    frags(s % NST, 1, fa1, fb1);
    mfmas(fa0, fb0);
    if (s + 1 < k_steps) {
      wait_stages(k_steps - 2 - s);  // stages s + 2 .. k_steps - 1 may still be in flight
      barrier_lds();
      frags((s + 1) % NST, 0, fa0, fb0);
    }
    mfmas(fa1, fb1);
  }

  // ---- epilogue: kRowsEpi rows at a time -> LDS -> pack / round / store
  // lane holds out[wm + 32i + 8*(e/4) + 4*(lane/32) + e%4][wn + 32j + lane%32]
  __syncthreads();  // the last stage's fragment reads are done before the union is reused
  constexpr int kRoundsPerWaveRow = kWM / kRowsEpi;  // rounds over one wave row's 128 rows
#pragma unroll
  for (int q = 0; q < BM / kRowsEpi; ++q) {
    if (wave / kWavesN == q / kRoundsPerWaveRow) {  // the waves holding this round's rows
#pragma unroll
      for (int ii = 0; ii < kRowsEpi / 32; ++ii) {
        const int i = (q % kRoundsPerWaveRow) * (kRowsEpi / 32) + ii;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sm.c[32 * ii + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][wn + 32 * j + (lane & 31)] = acc[i][j][e];
      }
    }
    __syncthreads();
    // kRowsEpi rows x BN / 16 groups of 16 columns
#pragma unroll
    for (int it = 0; it < kRowsEpi * (BN / 16) / kThreads; ++it) {
      const int g = tid + kThreads * it;
      const int r = g / (BN / 16), cg = g % (BN / 16);
      const int64_t t = m0 + kRowsEpi * q + r;
      const int n = n0 + 16 * cg;
      if (t >= a.tokens || n >= n_total) continue;
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = sm.c[r][16 * cg + i];
      store_group(a, t, n, v);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_ced_project(const uint16_t *h, int64_t tokens, int hidden, int n_layers, const uint16_t *w_kv,
                              const uint16_t *w_z, uint8_t *codes, uint8_t *scales, uint16_t *z, float *c_f32,
                              hipStream_t st) {
  if (tokens == 0 || n_layers == 0) return hipSuccess;
  CedArgs a{h, w_kv, w_z, tokens, hidden, n_layers, codes, scales, z, c_f32};
  const int n_total = n_layers * (w_z != nullptr ? kLatent + kIdxDim : kLatent);
  constexpr int kBN = 256, kStages = 4;
  const dim3 grid((n_total + kBN - 1) / kBN, (unsigned)((tokens + BM - 1) / BM));
  timer_before(kKernCedProject, st);
  ced_kernel<kBN, kStages><<<grid, dim3(2 * kBN), 0, st>>>(a);
  timer_after(kKernCedProject, st);
  return hipGetLastError();
}

}  // namespace csa2
