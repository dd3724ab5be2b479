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
// A workgroup computes a 256 x 128 output tile with 4 waves (128 x 64 each,
// 4 x 2 MFMA tiles of 32 x 32), k-steps of 64 staged through one LDS buffer
// with a register prefetch of the next step (the loads have a whole k-step of
// 32 MFMAs per wave to arrive); two workgroups share a CU, and the tiles are
// dealt so that each XCD's L2 serves a block of neighbouring tiles.  The epilogue parks the fp32 tile in
// LDS and packs each 16-channel group of C straight to E2M1 + E4M3 (the same
// rounding rules as the standalone pack) and rounds Z to bf16, so C never
// reaches HBM in fp32 (unless the optional debug copy is asked for).
#include "common.h"
#include "kernels.h"

namespace csa2 {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kLdA = BK + 8;   // bf16 per LDS row (pad breaks bank conflicts)
constexpr int kWM = 128, kWN = 64;  // wave tile: 4 x 2 MFMA tiles of 32 x 32
constexpr int kLdC = BN + 4;   // fp32 per epilogue row (128 rows at a time)
constexpr int kGroupM = 8;     // row tiles an XCD sweeps across the columns together
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

// Row n of the combined weight matrix, or null for a Z row without weights.
__device__ __forceinline__ const uint16_t *weight_row(const CedArgs &a, int n) {
  const int npl = per_layer(a.w_z);
  const int l = n / npl, c = n % npl;
  if (c < kLatent) return a.w_kv + ((size_t)l * kLatent + c) * a.hidden;
  if (a.w_z == nullptr) return nullptr;
  return a.w_z + ((size_t)l * kIdxDim + (c - kLatent)) * a.hidden;
}

union SmemCed {
  struct {
    uint16_t a[1][BM][kLdA];  // one buffer: the next k-step waits in registers
    uint16_t b[1][BN][kLdA];
  } ab;
  float c[kWM][kLdC];  // half of the output tile at a time in the epilogue
};

// 256 x 128 output tile per workgroup, 4 waves of 128 x 64 (8 independent
// 32 x 32 accumulators per wave: each A fragment feeds 2 MFMAs, each B
// fragment 4); two workgroups fit one CU.
__global__ void __launch_bounds__(256) ced_kernel(CedArgs a) {
  __shared__ __attribute__((aligned(16))) SmemCed sm;
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
  const int wm = (wave >> 1) * kWM, wn = (wave & 1) * kWN;

  // global -> register staging: a thread loads rows (tid / 8) + 32 i of A (i < 8) and of
  // B (i < 4), 16-byte column chunk tid % 8
  const int ld_row = tid >> 3, ld_col = 8 * (tid & 7);
  const uint16_t *a_src[8];
  const uint16_t *b_src[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + ld_row + 32 * i;
    a_src[i] = m < a.tokens ? a.h + m * a.hidden + ld_col : nullptr;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + ld_row + 32 * i;
    b_src[i] = n < n_total ? weight_row(a, n) : nullptr;
    if (b_src[i]) b_src[i] += ld_col;
  }
  uint4 ra[8], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4 *>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = b_src[i] ? *reinterpret_cast<const uint4 *>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4 *>(&sm.ab.a[buf][ld_row + 32 * i][ld_col]) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&sm.ab.b[buf][ld_row + 32 * i][ld_col]) = rb[i];
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int k_steps = a.hidden / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int ks = 0; ks < k_steps; ++ks) {
    const int buf = 0;
    if (ks + 1 < k_steps) fetch((ks + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(&sm.ab.a[buf][wm + 32 * i + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8 *>(&sm.ab.b[buf][wn + 32 * j + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    // scheduling: spread the k-step's 24 LDS reads and 12 global loads between its 32 MFMAs
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __syncthreads();  // every wave is done reading the tile
    if (ks + 1 < k_steps) stash(0);
    __syncthreads();
  }

  // ---- epilogue: 128 rows at a time -> LDS -> pack / round / store
  // lane holds out[wm + 32i + 8*(e/4) + 4*(lane/32) + e%4][wn + 32j + lane%32]
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wave >> 1) == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sm.c[32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][wn + 32 * j + (lane & 31)] = acc[i][j][e];
    }
    __syncthreads();
    // 128 rows x 8 groups of 16 columns = 1024 groups, 4 per thread
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int g = tid + 256 * it;
      const int r = g >> 3, cg = g & 7;
      const int64_t t = m0 + kWM * half + r;
      const int n = n0 + 16 * cg;
      if (t >= a.tokens || n >= n_total) continue;
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = sm.c[r][16 * cg + i];
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
      } else if (a.z != nullptr && a.w_z != nullptr) {
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
  const dim3 grid((n_total + BN - 1) / BN, (unsigned)((tokens + BM - 1) / BM));
  timer_before(kKernCedProject, st);
  ced_kernel<<<grid, dim3(256), 0, st>>>(a);
  timer_after(kKernCedProject, st);
  return hipGetLastError();
}

}  // namespace csa2
