// Batched bf16 GEMM on gfx950 MFMA with fp32 accumulation, for the dense
// projections of the training path: the key and value up-projections
// k = c W^UK_g, v = c W^UV_g, the latent gradient dc = dk W^UK^T + dv W^UV^T and
// the weight gradients dW_g = c^T dY_g.
//
// C[z][m][n] (+)= sum_k A[z][m][k] B[z][k][n].  Each operand is either
// K-contiguous (element (mn, k) at mn*ld + k, with k split into groups of
// kgrp elements kgrp_stride apart, so a K index can run over the groups of a
// [G][r][d] weight) or MN-contiguous (element (mn, k) at k*ld + mn).
// Workgroup tile GT x GT (128, or 64 when the 128 tiles would leave most CUs
// idle), K step 32; wave w computes the GT/2 x GT/2 block (w/2, w%2) as
// GT/64 x GT/64 MFMA 32x32x16 blocks.  Tiles are staged in LDS through
// registers, double-buffered, one barrier per K step.  MFMA operand layouts:
// A lane l holds A[m=l%32][k=8(l/32)+j]; B lane l holds B[k=8(l/32)+j][n=l%32];
// D lane l reg i holds D[8(i/4)+4(l/32)+i%4][l%32].  A K-contiguous tile is
// read with ds_read_b128 (8 consecutive k of one row); an MN-contiguous tile
// with two ds_read_b64_tr_b16 (within each 16-lane group lane i receives
// element i%4 of the 8-byte loads of lanes 4e + i/4: four k rows of one mn).
#include "device_common.h"
#include "qkmla_internal.h"

namespace qkmla {

namespace {

constexpr int kGK = 32;                    // K step
constexpr int kKcPitch = kGK * 2 + 16;     // 80 B: K-contiguous tile row (one mn)

template <int GT>
struct TileGeom {
  static constexpr int kMnPitch = GT * 2 + 16;  // MN-contiguous tile row (one k): 272 B at 128
  static constexpr int kStageBytes =
      GT * kKcPitch > kGK * kMnPitch ? GT * kKcPitch : kGK * kMnPitch;
  static constexpr int kPerThread = GT / 64;    // 16-byte chunks per thread and operand
};

template <bool KC, int GT>
struct OperandTile {
  static constexpr int kMnPitch = TileGeom<GT>::kMnPitch;
  static constexpr int kRowChunks = GT / 8;  // chunks per MN-contiguous k row
  // 4 GT chunks of 16 B per tile, GT/64 per thread.
  // K-contiguous: chunk c -> row mn = c/4, k = 8*(c%4).
  // MN-contiguous: chunk c -> k row = c/(GT/8), mn = 8*(c%(GT/8)).
  __device__ static uint4 load(const GemmOperand& o, int z, int mn0, int MN, int k0, int K,
                               int c) {
    const uint16_t* base = o.p + (size_t)z * o.batch_stride;
    if constexpr (KC) {
      const int mn = min(mn0 + c / 4, MN - 1);
      const int k = k0 + 8 * (c % 4);
      if (k >= K) return make_uint4(0, 0, 0, 0);
      const size_t off = (size_t)mn * o.ld + (size_t)(k / o.kgrp) * o.kgrp_stride + k % o.kgrp;
      return *(const uint4*)(base + off);
    } else {
      const int k = k0 + c / kRowChunks;
      const int mn = mn0 + 8 * (c % kRowChunks);
      if (k >= K || mn >= MN) return make_uint4(0, 0, 0, 0);
      return *(const uint4*)(base + (size_t)k * o.ld + mn);
    }
  }
  __device__ static void store(char* st, int c, uint4 v) {
    if constexpr (KC) *(uint4*)(st + (c / 4) * kKcPitch + 16 * (c % 4)) = v;
    else *(uint4*)(st + (c / kRowChunks) * kMnPitch + 16 * (c % kRowChunks)) = v;
  }
  // MFMA operand for rows mn0 .. mn0+31 of the tile, k-step s (16 k).
  __device__ static bf16x8 read(const char* st, int mn0, int s, int lane) {
    const int hf = lane >> 5;
    if constexpr (KC) {
      return *(const bf16x8*)(st + (mn0 + (lane & 31)) * kKcPitch + 2 * (16 * s + 8 * hf));
    } else {
      const int s16 = lane & 15, grp = (lane >> 4) & 1;
      const char* p = st + (16 * s + 8 * hf + (s16 >> 2)) * kMnPitch +
                      2 * (mn0 + 16 * grp + 4 * (s16 & 3));
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, p));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, p + 4 * kMnPitch));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

template <bool A_KC, bool B_KC, int GT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int kStageBytes = TileGeom<GT>::kStageBytes;
  constexpr int kPer = TileGeom<GT>::kPerThread;
  constexpr int kBlk = GT / 64;  // MFMA blocks per wave along m and n
  __shared__ __attribute__((aligned(16))) char a_st[2][kStageBytes];
  __shared__ __attribute__((aligned(16))) char b_st[2][kStageBytes];
  using TA = OperandTile<A_KC, GT>;
  using TB = OperandTile<B_KC, GT>;
  const int n0 = blockIdx.x * GT, m0 = blockIdx.y * GT, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[kBlk][kBlk];
#pragma unroll
  for (int i = 0; i < kBlk; ++i)
#pragma unroll
    for (int j = 0; j < kBlk; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (g.K + kGK - 1) / kGK;
  uint4 ra[kPer], rb[kPer];
  auto load = [&](int kt) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      ra[u] = TA::load(g.A, z, m0, g.M, kt * kGK, g.K, tid + 256 * u);
      rb[u] = TB::load(g.B, z, n0, g.N, kt * kGK, g.K, tid + 256 * u);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      TA::store(a_st[buf], tid + 256 * u, ra[u]);
      TB::store(b_st[buf], tid + 256 * u, rb[u]);
    }
  };
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8 av[kBlk], bv[kBlk];
#pragma unroll
      for (int i = 0; i < kBlk; ++i) av[i] = TA::read(a_st[buf], GT / 2 * wm + 32 * i, s, lane);
#pragma unroll
      for (int j = 0; j < kBlk; ++j) bv[j] = TB::read(b_st[buf], GT / 2 * wn + 32 * j, s, lane);
#pragma unroll
      for (int i = 0; i < kBlk; ++i)
#pragma unroll
        for (int j = 0; j < kBlk; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // lane l reg r of block (i, j): row (GT/2)wm + 32i + 8(r/4) + 4(l/32) + r%4,
  // col (GT/2)wn + 32j + l%32
  float* C = g.C + (size_t)z * g.c_batch_stride;
  const int hf = lane >> 5;
#pragma unroll
  for (int j = 0; j < kBlk; ++j) {
    const int n = n0 + GT / 2 * wn + 32 * j + (lane & 31);
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < kBlk; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + GT / 2 * wm + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (m >= g.M) continue;
        float* p = C + (size_t)m * g.ldc + n;
        *p = g.accumulate ? *p + acc[i][j][r] : acc[i][j][r];
      }
  }
}

}  // namespace

template <int GT>
static hipError_t launch_gemm_gt(const GemmArgs& g, bool a_kc, bool b_kc, int batch,
                                 hipStream_t s) {
  const dim3 grid((g.N + GT - 1) / GT, (g.M + GT - 1) / GT, batch);
  // the three layout pairs the training path uses
  if (a_kc && b_kc)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, GT>), grid, dim3(256), 0, s, g);
  else if (a_kc)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, GT>), grid, dim3(256), 0, s, g);
  else if (!b_kc)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, GT>), grid, dim3(256), 0, s, g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_kc, bool b_kc, int batch, hipStream_t s) {
  // 128 x 128 tiles while they give every CU a workgroup, else 64 x 64
  const int64_t big = (int64_t)((g.N + 127) / 128) * ((g.M + 127) / 128) * batch;
  if (big >= 256) return launch_gemm_gt<128>(g, a_kc, b_kc, batch, s);
  return launch_gemm_gt<64>(g, a_kc, b_kc, batch, s);
}

}  // namespace qkmla
