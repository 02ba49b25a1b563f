// Static weight absorption and cache append for QK-Normed MLA.
//
// absorb: W~_g^T[i][j] = gamma_q[j] * gamma_k[j] * W^UK[g][i][j]
//   ("QK-Normed MLA: QK normalization without full key caching", technical
//   summary, Methodology: Static Weight Absorption -- gamma_k and gamma_q move
//   into the query-side projection).
// append: per new token, copy the latent row, cache alpha^k_g = 1/S(c W^UK_g)
//   for every KV group (Methodology: Dynamic Scalar Caching and Cache Layout),
//   and store the RoPE key RMS-normalised on its own and rotated
//   (Methodology: Blockwise Normalization).
#include "device_common.h"
#include "qkmla_internal.h"

namespace qkmla {

template <typename T>
__global__ __launch_bounds__(256) void absorb_kernel(const float* __restrict__ w_uk,
                                                     const float* __restrict__ gq,
                                                     const float* __restrict__ gk,
                                                     T* __restrict__ out, int64_t n, int dc,
                                                     int qk_norm) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float w = w_uk[i];
  if (qk_norm) {
    int j = (int)(i % dc);
    w *= gq[j] * gk[j];
  }
  Elem<T>::store(out, (size_t)i, w);
}

hipError_t launch_absorb(const Cfg& c, const float* w_uk, const float* gq, const float* gk,
                         void* w_qabs, hipStream_t s) {
  int64_t n = (int64_t)c.G * c.r * c.dc;
  dim3 grid((unsigned)((n + 255) / 256));
  if (c.dtype == QKMLA_BF16)
    absorb_kernel<uint16_t><<<grid, 256, 0, s>>>(w_uk, gq, gk, (uint16_t*)w_qabs, n, c.dc,
                                                 c.qk_norm);
  else
    absorb_kernel<float><<<grid, 256, 0, s>>>(w_uk, gq, gk, (float*)w_qabs, n, c.dc, c.qk_norm);
  return hipGetLastError();
}

// Copy the latent rows of tokens tok0..tok0+ntok-1 and write their RoPE keys,
// RMS-normalised on their own (QK-norm) and rotated by the cache row.  A
// sequence whose rows would fall outside the cache gets no writes and sets
// QKMLA_DEV_BAD_POSITION.  Called by every thread of the block: each
// wavefront takes whole tokens (wave w: tokens w, w + waves, ...), so no
// token waits on a block barrier; a bf16 row of r = 512 is one 16-byte piece
// per lane.
template <typename T>
__device__ void copy_rows_and_rope(int tok0, int ntok, int batch, int n_new,
                                   const T* __restrict__ c_new, const T* __restrict__ kr_new,
                                   const float* __restrict__ gkr,
                                   const int32_t* __restrict__ positions, const Paging pg,
                                   T* __restrict__ lat, T* __restrict__ rope, int32_t* status,
                                   int r, int dr, float eps, const RopeFreq& rf, int qk_norm) {
  const int T_total = batch * n_new;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  // 16-byte pieces of a latent row, when rows are whole pieces and aligned
  const bool vec = (r * sizeof(T)) % 16 == 0 && ((uintptr_t)c_new % 16) == 0 &&
                   ((uintptr_t)lat % 16) == 0;
  const int n16 = (int)(r * sizeof(T) / 16);
  for (int k = wave; k < ntok; k += nwaves) {
    const int tok = tok0 + k;
    if (tok >= T_total) break;
    const int b = tok / n_new, i = tok % n_new;
    const int pos0 = positions[b];
    if (pos0 < 0 || (int64_t)pos0 + n_new > pg.capacity()) {
      if (lane == 0 && i == 0 && status) atomicOr(status, QKMLA_DEV_BAD_POSITION);
      continue;
    }
    const int row = pos0 + i;
    const int64_t prow = pg.phys_row(b, row);
    if (prow < 0) {
      if (lane == 0 && status) atomicOr(status, QKMLA_DEV_BAD_PAGE);
      continue;
    }
    if (vec) {
      const uint4* src = (const uint4*)(c_new + (size_t)tok * r);
      uint4* dst = (uint4*)(lat + (size_t)prow * r);
      for (int e = lane; e < n16; e += 64) dst[e] = src[e];
    } else {
      const T* src = c_new + (size_t)tok * r;
      T* dst = lat + (size_t)prow * r;
      for (int e = lane; e < r; e += 64) dst[e] = src[e];
    }
    // RoPE key: optional RMSNorm over d_r, then rotate pairs by row position.
    const T* ks = kr_new + (size_t)tok * dr;
    float scale = 1.f;
    if (qk_norm) {
      float acc = 0.f;
      for (int e = lane; e < dr; e += 64) {
        const float v = Elem<T>::load(ks, e);
        acc += v * v;
      }
      scale = 1.0f / sqrtf(wave_sum(acc) / (float)dr + eps);
    }
    T* rdst = rope + (size_t)prow * dr;
    for (int pi = lane; pi < dr / 2; pi += 64) {
      float x0 = Elem<T>::load(ks, 2 * pi), x1 = Elem<T>::load(ks, 2 * pi + 1);
      if (qk_norm) {
        x0 = x0 * scale * gkr[2 * pi];
        x1 = x1 * scale * gkr[2 * pi + 1];
      }
      float cs_, sn_;
      rope_cos_sin_freq(row, rf.f[pi], &cs_, &sn_);
      Elem<T>::store(rdst, 2 * pi, x0 * cs_ - x1 * sn_);
      Elem<T>::store(rdst, 2 * pi + 1, x0 * sn_ + x1 * cs_);
    }
  }
}

// One workgroup per (block of kAppendTok new tokens, duty).  Duty y < G
// computes alpha^k for group y; duty y == G (or 0 in plain mode) copies the
// latent rows and writes the normalised, rotated RoPE key.
constexpr int kAppendTok = 8;
constexpr int kMaxR = 1024;
constexpr int kMaxDc = 1024;

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(
    int batch, int n_new, const T* __restrict__ c_new, const T* __restrict__ kr_new,
    const float* __restrict__ w_uk, const float* __restrict__ gkr,
    const int32_t* __restrict__ positions, const Paging pg, T* __restrict__ lat,
    T* __restrict__ rope, float* __restrict__ alpha, int32_t* status, int G, int r, int dc, int dr,
    float eps, const RopeFreq rf, int qk_norm) {
  __shared__ float cs[kAppendTok * kMaxR];
  __shared__ float ksq[kAppendTok];
  const int T_total = batch * n_new;
  const int tok0 = blockIdx.x * kAppendTok;
  const int duty = blockIdx.y;
  const bool copy_duty = qk_norm ? (duty == G) : (duty == 0);
  const int tid = threadIdx.x;

  if (copy_duty) {
    copy_rows_and_rope<T>(tok0, kAppendTok, batch, n_new, c_new, kr_new, gkr, positions, pg,
                          lat, rope, status, r, dr, eps, rf, qk_norm);
    return;
  }

  // alpha^k for group g = duty over up to kAppendTok tokens.
  const int g = duty;
  int ntok = min(kAppendTok, T_total - tok0);
  for (int k = 0; k < ntok; ++k) {
    const T* src = c_new + (size_t)(tok0 + k) * r;
    for (int e = tid; e < r; e += blockDim.x) cs[k * kMaxR + e] = Elem<T>::load(src, e);
  }
  if (tid < kAppendTok) ksq[tid] = 0.f;
  __syncthreads();
  const float* W = w_uk + (size_t)g * r * dc;
  // Work items (token k, output column j).
  float part[kAppendTok];
#pragma unroll
  for (int k = 0; k < kAppendTok; ++k) part[k] = 0.f;
  for (int j = tid; j < dc; j += blockDim.x) {
    float acc[kAppendTok];
#pragma unroll
    for (int k = 0; k < kAppendTok; ++k) acc[k] = 0.f;
    for (int i = 0; i < r; ++i) {
      float w = W[(size_t)i * dc + j];
#pragma unroll
      for (int k = 0; k < kAppendTok; ++k) acc[k] += cs[k * kMaxR + i] * w;
    }
#pragma unroll
    for (int k = 0; k < kAppendTok; ++k) part[k] += acc[k] * acc[k];
  }
#pragma unroll
  for (int k = 0; k < kAppendTok; ++k) {
    float v = wave_sum(part[k]);
    if ((tid & 63) == 0) atomicAdd(&ksq[k], v);
  }
  __syncthreads();
  if (tid < ntok) {
    int tok = tok0 + tid;
    int b = tok / n_new, i = tok % n_new;
    int pos0 = positions[b];
    bool bad = pos0 < 0 || (int64_t)pos0 + n_new > pg.capacity();
    const int64_t prow = bad ? -1 : pg.phys_row(b, pos0 + i);
    if (prow >= 0) {
      float a = 1.0f / sqrtf(ksq[tid] / (float)dc + eps);
      alpha[(size_t)prow * G + g] = a;
    }
  }
}

// bf16 caches: one workgroup per (32 TB new tokens, duty).  Duty y < G
// computes alpha^k of group y on MFMA; duties y >= G (y == 0 .. TB - 1 in
// plain mode) copy 32 latent rows each and write their RoPE keys.
//   k^T[n][t] = sum_i W^UK_g[i][n] c_t[i]          (mfma_f32_32x32x16_bf16)
//   alpha^k_{t,g} = 1 / sqrt(mean_n k^T[n][t]^2 + eps)
// The four waves take output dims n in blocks of 32 (wave w: blocks w, w+4)
// for all TB token blocks, so each W^UK_g chunk staged in LDS serves 32 TB
// tokens.  W^UK stays accurate to about 2^-16: each weight is split into
// hi = bf16(W) and lo = bf16(W - hi), and both products with the bf16
// latent are exact, accumulated in fp32.  The chunks of 32 rows are double
// buffered: chunk k + 1's weights and latent operands are loaded into
// registers while chunk k is converted into the LDS buffer k % 2 and
// multiplied, so one barrier per chunk suffices and the loads' latency hides
// behind the MFMAs.  The A operand W^T[n][k] comes from ds_read_b64_tr_b16 of
// the row-major hi / lo tiles: in each 16-lane group lane i receives element
// i%4 of the 8-byte loads of lanes 4e + i/4.
// MFMA 32x32x16 layouts: A lane l holds A[m=l%32][k=8(l/32)+j]; B lane l
// holds B[k=8(l/32)+j][n=l%32]; D lane l reg i holds D[8(i/4)+4(l/32)+i%4][l%32].
constexpr int kAlphaChunk = 32;
constexpr int kAlphaMaxDc = 256;
// WQ: W^UK quads per thread and chunk, kAlphaChunk * d_c / 4 / 256 rounded up
// to 4 or 8 (d_c <= 128 or <= 256).
// (with d_c <= 128, two workgroups share a CU: measured 420 against 560 us
// for 64 Ki tokens with one, the phases of one workgroup (loads, conversion,
// barrier, MFMAs) then overlapping with the other's)
template <int TB, int WQ>
__global__ __launch_bounds__(256, WQ == 4 ? 2 : 1) void append_bf16_kernel(
    int batch, int n_new, const uint16_t* __restrict__ c_new, const uint16_t* __restrict__ kr_new,
    const float* __restrict__ w_uk, const float* __restrict__ gkr,
    const int32_t* __restrict__ positions, const Paging pg, uint16_t* __restrict__ lat,
    uint16_t* __restrict__ rope, float* __restrict__ alpha, int32_t* status, int G, int r,
    int dc, int dr, float eps, const RopeFreq rf, int qk_norm) {
  __shared__ __attribute__((aligned(16))) uint16_t w_hi[2][kAlphaChunk][kAlphaMaxDc];
  __shared__ __attribute__((aligned(16))) uint16_t w_lo[2][kAlphaChunk][kAlphaMaxDc];
  __shared__ float ssq[4][32 * TB];
  const int T_total = batch * n_new;
  const int tok0 = blockIdx.x * 32 * TB;
  const int duty = blockIdx.y;
  const int copy0 = qk_norm ? G : 0;
  if (duty >= copy0) {
    copy_rows_and_rope<uint16_t>(tok0 + 32 * (duty - copy0), 32, batch, n_new, c_new, kr_new, gkr,
                                 positions, pg, lat, rope, status, r, dr, eps, rf, qk_norm);
    return;
  }
  const int g = duty;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, t = lane & 31;
  const int nblk = dc / 32;  // 1..8
  const int nq = dc / 4;     // column quads of a W^UK row
  // A operand through the transposing read: this lane loads row e (+4) of the
  // K-step's 16, columns 4q..4q+3 of its 16-column half
  const int q16 = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
  const int a_row = 8 * (q16 >> 1) + e;
  const int a_col = 16 * (q16 & 1) + 4 * q;
  const float* W = w_uk + (size_t)g * r * dc;
  // B operand: token tb*32 + t's latent row, elements 8 hf .. 8 hf + 7 of each
  // K-step (rows past the last token repeat it)
  const uint16_t* crow[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
    crow[tb] = c_new + (size_t)min(tok0 + 32 * tb + t, T_total - 1) * r + hf * 8;
  f32x16 acc[2][TB];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[bi][tb][j] = 0.f;
  struct Chunk {
    f32x4 w[WQ];
    bf16x8 c[TB][kAlphaChunk / 16];
  };
  auto load = [&](int k0, Chunk& ch) {
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      const int i = tid + 256 * u;  // the test is uniform: i < 256 (u + 1) <= chunk quads
      if (i < kAlphaChunk * nq) ch.w[u] = *(const f32x4*)(W + (size_t)(k0 + i / nq) * dc + (i % nq) * 4);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int ks = 0; ks < kAlphaChunk / 16; ++ks)
        ch.c[tb][ks] = *(const bf16x8*)(crow[tb] + k0 + ks * 16);
  };
  Chunk cur, nxt;
  load(0, cur);
  const int nchunk = r / kAlphaChunk;
  for (int kc = 0; kc < nchunk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nchunk) load((kc + 1) * kAlphaChunk, nxt);
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      const int i = tid + 256 * u;
      if (i < kAlphaChunk * nq) {
        const int row = i / nq, c4 = (i % nq) * 4;
        bf16x4 hi, lo;  // hardware round-to-nearest-even conversions
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi[j] = (__bf16)cur.w[u][j];
          lo[j] = (__bf16)(cur.w[u][j] - (float)hi[j]);
        }
        *(bf16x4*)&w_hi[buf][row][c4] = hi;
        *(bf16x4*)&w_lo[buf][row][c4] = lo;
      }
    }
    // chunk kc is in LDS buffer buf; every wave is past chunk kc - 1's reads
    // of the other buffer (the previous barrier), which chunk kc + 1 rewrites
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kAlphaChunk / 16; ++ks) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int blk = wave + 4 * bi;
        if (blk < nblk) {
          const int rr = ks * 16 + a_row, cc = blk * 32 + a_col;
          const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &w_hi[buf][rr][cc]));
          const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &w_hi[buf][rr + 4][cc]));
          const bf16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &w_lo[buf][rr][cc]));
          const bf16x4 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &w_lo[buf][rr + 4][cc]));
          const bf16x8 ah = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          const bf16x8 alo = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[bi][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, cur.c[tb][ks], acc[bi][tb], 0, 0, 0);
            acc[bi][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, cur.c[tb][ks], acc[bi][tb], 0, 0, 0);
          }
        }
      }
    }
    cur = nxt;
  }
  // lane l holds k^T[n][t] for 16 dims n of each of its blocks and token t of
  // each token block; the two halves of a column (lanes l, l ^ 32) meet by a
  // half-wave swap
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    float sq = 0.f;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int j = 0; j < 16; ++j) sq += acc[bi][tb][j] * acc[bi][tb][j];
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sq), __float_as_uint(sq),
                                                     false, false);
    sq = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (hf == 0) ssq[wave][32 * tb + t] = sq;
  }
  __syncthreads();
  if (tid < 32 * TB) {
    const int tok = tok0 + tid;
    if (tok < T_total) {
      const int b = tok / n_new, i = tok % n_new;
      const int pos0 = positions[b];
      const bool bad = pos0 < 0 || (int64_t)pos0 + n_new > pg.capacity();
      const int64_t prow = bad ? -1 : pg.phys_row(b, pos0 + i);
      if (prow >= 0) {
        const float ss = ssq[0][tid] + ssq[1][tid] + ssq[2][tid] + ssq[3][tid];
        alpha[(size_t)prow * G + g] = 1.0f / sqrtf(ss / (float)dc + eps);
      }
    }
  }
}

// Few new tokens (the decode step's append): alpha^k on VALU with every
// weight load in flight at once.  One block of 1024 threads per (chunk of up
// to kStepTok tokens, group g).  Thread (row group rg, column quad c4) owns
// columns 4 c4..4 c4+3 of W^UK_g (fp32, 16-byte loads) and rows rg, rg + RG,
// ... (RG = 1024 / (d_c / 4) row groups); it accumulates k over its rows for
// every token of the chunk, the two row groups of a wavefront meet by a
// cross-lane add and the wavefronts in LDS, then k^2 is summed over d_c.
// The copy of the latent rows and the RoPE key is the extra duty y = G of
// the same launch.  W^UK_g (fp32 [r][d_c]) is read once per chunk: for the
// 128-dim groups of the DeepSeek-V3-like layer, 256 KB per block, one round
// of loads.
constexpr int kStepTok = 4;
constexpr int kStepThreads = 1024;
constexpr int kStepMaxDc = 256;
constexpr int kStepMaxRowsPerThread = 16;  // r / RG

// DC, R > 0: the layer shape fixed at compile time (every loop below has a
// static trip count, so all of its loads go out together); 0: read d_c and r
// from the arguments.
template <typename T, int DC, int R>
__global__ __launch_bounds__(kStepThreads) void append_step_kernel(
    int batch, int n_new, const T* __restrict__ c_new, const T* __restrict__ kr_new,
    const float* __restrict__ w_uk, const float* __restrict__ gkr,
    const int32_t* __restrict__ positions, const Paging pg, T* __restrict__ lat,
    T* __restrict__ rope, float* __restrict__ alpha, int32_t* status, int G, int r, int dc, int dr,
    float eps, const RopeFreq rf, int qk_norm) {
  __shared__ float cs[kStepTok][kMaxR];                         // 16 KB
  __shared__ float kp[kStepThreads / 64][kStepTok][kStepMaxDc];  // 64 KB
  __shared__ float sqv[kStepTok][kStepMaxDc];
  const int T_total = batch * n_new;
  const int tok0 = blockIdx.x * kStepTok;
  const int ntok = min(kStepTok, T_total - tok0);
  const int duty = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (qk_norm ? duty == G : duty == 0) {
    copy_rows_and_rope<T>(tok0, kStepTok, batch, n_new, c_new, kr_new, gkr, positions, pg, lat,
                          rope, status, r, dr, eps, rf, qk_norm);
    return;
  }
  const int g = duty;
  if constexpr (DC > 0) dc = DC;
  if constexpr (R > 0) r = R;
  const int nq = dc / 4;               // column quads
  const int RG = kStepThreads / nq;    // row groups
  const int rg = tid / nq, c4 = tid % nq;
  const int rows = r / RG;             // rows per thread (<= kStepMaxRowsPerThread)
  const float* W = w_uk + (size_t)g * r * dc + 4 * c4;
  // The loads go out in the order they are needed (they complete in that
  // order): the new latent rows, the tokens' positions, then W^UK_g, so the
  // LDS copy of the rows and the row lookup do not wait for the weights.
  constexpr int kCs = R > 0 ? (kStepTok * R + kStepThreads - 1) / kStepThreads : 1;
  T cv[kCs];  // raw elements, converted when they go to LDS (after the weights' loads)
  if constexpr (R > 0) {
#pragma unroll
    for (int u = 0; u < kCs; ++u) {  // unconditional loads (clamped), selected later
      const int i = tid + u * kStepThreads;
      cv[u] = c_new[(size_t)tok0 * R + min(i, ntok * R - 1)];
    }
  } else {
    for (int i = tid; i < kStepTok * r; i += kStepThreads) {
      const int k = i / r, e = i % r;
      cs[k][e] = k < ntok ? Elem<T>::load(c_new, (size_t)(tok0 + k) * r + e) : 0.f;
    }
  }
  // Wavefront k writes token k's alpha: its position (and, for a paged cache,
  // the block-table entry) through scalar loads, which the weights' vector
  // loads in flight do not hold up.
  const int wv_id = __builtin_amdgcn_readfirstlane(wave);
  const __attribute__((address_space(4))) int32_t* pos_s =
      (const __attribute__((address_space(4))) int32_t*)positions;
  const int pos0 = wv_id < ntok ? pos_s[(tok0 + wv_id) / n_new] : 0;
  // Branch-free: rows past r / RG re-read the last one and are not summed.
  f32x4 wv[kStepMaxRowsPerThread];
#pragma unroll
  for (int n = 0; n < kStepMaxRowsPerThread; ++n)
    wv[n] = *(const f32x4*)(W + (size_t)(rg + min(n, rows - 1) * RG) * dc);
  if constexpr (R > 0) {
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the first use
#pragma unroll
    for (int u = 0; u < kCs; ++u) {
      const int i = tid + u * kStepThreads;
      if (i < kStepTok * R) cs[i / R][i % R] = i / R < ntok ? Elem<T>::load(cv, u) : 0.f;
    }
  }
  int64_t prow = -1;
  if (wv_id < ntok) {
    const int tok = tok0 + wv_id;
    const int b = tok / n_new, i = tok % n_new;
    const bool bad = pos0 < 0 || (int64_t)pos0 + n_new > pg.capacity();
    if (!bad) {
      const int t = pos0 + i, blk = t / pg.page_size;
      int page = b;
      if (pg.bt) {
        page = ((const __attribute__((address_space(4))) int32_t*)pg.bt)[(size_t)b * pg.max_blocks +
                                                                          blk];
        page = (page >= 0 && page < pg.num_pages) ? page : -1;
      }
      prow = page < 0 ? -1 : (int64_t)page * pg.page_size + (t - blk * pg.page_size);
    }
  }
  __syncthreads();
  f32x4 acc[kStepTok];
#pragma unroll
  for (int k = 0; k < kStepTok; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < kStepMaxRowsPerThread; ++n)
    if (n < rows) {
      const int i = rg + n * RG;
#pragma unroll
      for (int k = 0; k < kStepTok; ++k) acc[k] += cs[k][i] * wv[n];
    }
  // the two row groups of a wavefront (nq = 32: lanes l and l ^ 32) meet here
  // when a wavefront spans two of them
  const bool pair = nq == 32;
#pragma unroll
  for (int k = 0; k < kStepTok; ++k) {
    f32x4 v = acc[k];
    if (pair) {  // lanes l and l ^ 32: one half-wave swap each, no LDS round trip
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[q]),
                                                         __float_as_uint(v[q]), false, false);
        v[q] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
    }
    if (!pair || lane < 32) *(f32x4*)&kp[wave][k][4 * c4] = v;
  }
  __syncthreads();
  // k[t][j] = sum of the partials of the wavefronts that hold column j: all
  // of them when a wavefront spans two row groups (d_c = 128), else every
  // nq / 64-th one (a row group spans nq / 64 wavefronts).
  // Every sum has a fixed order, so the result is the same on every call.
  const int wstep = pair ? 1 : nq / 64;
  if constexpr (DC == 128) {  // the pair case: every wavefront holds every column
    if (tid < kStepTok * DC) {
      const int k = tid / DC, j = tid % DC;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kStepThreads / 64; ++w) v += kp[w][k][j];
      sqv[k][j] = v * v;
    }
  } else {
    for (int i = tid; i < kStepTok * dc; i += kStepThreads) {
      const int k = i / dc, j = i % dc;
      float v = 0.f;
      for (int w = pair ? 0 : (j / 4) / 64; w < kStepThreads / 64; w += wstep) v += kp[w][k][j];
      sqv[k][j] = v * v;
    }
  }
  __syncthreads();
  if (wave < ntok) {  // wavefront k: sum over d_c of token k's k^2
    float ss = 0.f;
    for (int j = lane; j < dc; j += 64) ss += sqv[wave][j];
    ss = wave_sum(ss);
    if (lane == 0 && prow >= 0) alpha[(size_t)prow * G + g] = 1.0f / sqrtf(ss / (float)dc + eps);
  }
}

hipError_t launch_append(const Cfg& c, int batch, int n_new, const void* c_new,
                         const void* k_rope_new, const float* w_uk, const float* gkr,
                         const int32_t* positions, const Paging& pg, void* lat, void* rope,
                         float* alpha, int32_t* status, hipStream_t s) {
  int T_total = batch * n_new;
  const RopeFreq rf = rope_freq(c.dr, c.base);
  // A decode step's few tokens: the latency-bound path with all of W^UK_g's
  // loads in flight; it reads W^UK as 16-byte vectors.
  const int nq = c.dc / 4;
  if (T_total <= 4 * kStepTok && c.dc % 4 == 0 && c.dc <= kStepMaxDc && (nq == 32 || nq % 64 == 0) &&
      c.r <= kMaxR && c.r % (kStepThreads / nq) == 0 &&
      c.r / (kStepThreads / nq) <= kStepMaxRowsPerThread &&
      ((uintptr_t)w_uk % 16 == 0 || !c.qk_norm)) {
    dim3 g1((unsigned)((T_total + kStepTok - 1) / kStepTok), c.qk_norm ? c.G + 1 : 1);
    const bool dsv3 = c.dc == 128 && c.r == 512;  // the DeepSeek-V3-like layer's shape
    if (c.dtype == QKMLA_BF16 && dsv3)
      append_step_kernel<uint16_t, 128, 512><<<g1, kStepThreads, 0, s>>>(
          batch, n_new, (const uint16_t*)c_new, (const uint16_t*)k_rope_new, w_uk, gkr,
          positions, pg, (uint16_t*)lat, (uint16_t*)rope, alpha, status, c.G, c.r, c.dc, c.dr,
          c.eps, rf, c.qk_norm);
    else if (c.dtype == QKMLA_BF16)
      append_step_kernel<uint16_t, 0, 0><<<g1, kStepThreads, 0, s>>>(
          batch, n_new, (const uint16_t*)c_new, (const uint16_t*)k_rope_new, w_uk, gkr,
          positions, pg, (uint16_t*)lat, (uint16_t*)rope, alpha, status, c.G, c.r, c.dc, c.dr,
          c.eps, rf, c.qk_norm);
    else
      append_step_kernel<float, 0, 0><<<g1, kStepThreads, 0, s>>>(
          batch, n_new, (const float*)c_new, (const float*)k_rope_new, w_uk, gkr, positions, pg,
          (float*)lat, (float*)rope, alpha, status, c.G, c.r, c.dc, c.dr, c.eps, rf, c.qk_norm);
    return hipGetLastError();
  }
  // The MFMA kernel reads latent rows and W^UK as 16-byte vectors.
  const bool vec_ok = ((uintptr_t)c_new % 16 == 0) && ((uintptr_t)w_uk % 16 == 0 || !c.qk_norm);
  if (c.dtype == QKMLA_BF16 && vec_ok && c.dc % 32 == 0 && c.dc <= kAlphaMaxDc &&
      c.r % kAlphaChunk == 0) {
    // Four token blocks per workgroup once the tokens give each group's
    // blocks the chip several times over: each W^UK_g chunk then serves 128
    // tokens instead of 32 (a quarter of the weight traffic and conversions).
    const bool wide = T_total >= 4096;
    const int per_wg = wide ? 128 : 32;
    dim3 g2((unsigned)((T_total + per_wg - 1) / per_wg),
            (c.qk_norm ? c.G : 0) + per_wg / 32);
#define QKMLA_APPEND_BF16(TB, WQ)                                                           \
  append_bf16_kernel<TB, WQ><<<g2, 256, 0, s>>>(batch, n_new, (const uint16_t*)c_new,         \
                                                (const uint16_t*)k_rope_new, w_uk, gkr,       \
                                                positions, pg, (uint16_t*)lat,                \
                                                (uint16_t*)rope, alpha, status, c.G, c.r,     \
                                                c.dc, c.dr, c.eps, rf, c.qk_norm)
    const bool narrow_dc = c.dc <= 128;
    if (wide && narrow_dc) QKMLA_APPEND_BF16(4, 4);
    else if (wide) QKMLA_APPEND_BF16(4, 8);
    else if (narrow_dc) QKMLA_APPEND_BF16(1, 4);
    else QKMLA_APPEND_BF16(1, 8);
#undef QKMLA_APPEND_BF16
    return hipGetLastError();
  }
  dim3 grid((unsigned)((T_total + kAppendTok - 1) / kAppendTok), c.qk_norm ? c.G + 1 : 1);
  if (c.dtype == QKMLA_BF16)
    append_kernel<uint16_t><<<grid, 256, 0, s>>>(
        batch, n_new, (const uint16_t*)c_new, (const uint16_t*)k_rope_new, w_uk, gkr, positions,
        pg, (uint16_t*)lat, (uint16_t*)rope, alpha, status, c.G, c.r, c.dc, c.dr, c.eps,
        rf, c.qk_norm);
  else
    append_kernel<float><<<grid, 256, 0, s>>>(
        batch, n_new, (const float*)c_new, (const float*)k_rope_new, w_uk, gkr, positions, pg,
        (float*)lat, (float*)rope, alpha, status, c.G, c.r, c.dc, c.dr, c.eps, rf,
        c.qk_norm);
  return hipGetLastError();
}

}  // namespace qkmla
