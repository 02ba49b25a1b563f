// Query preparation, the first kernel of a decode step.
//
// Per sequence b and head h (g = g(h), L_b = seq_lens[b]):
//   alpha^q_h = 1/S(q^C_h)                       (query-side dynamic scalar)
//   q~_h      = q^C_h W~_g                       (gammas already absorbed in W~)
//   q^R_h     = RoPE_{L_b-1}(RMSNorm_{gamma_q_rope}(q^R_h))
// ("QK-Normed MLA: QK normalization without full key caching", technical
// summary, Methodology: Static Weight Absorption, the decode-logit formula and
// Blockwise Normalization).  tau*log2(e) is folded into alpha^q and q^R so the
// decode kernel works in the exp2 domain.  In plain mode alpha^q = tau*log2(e)
// and q^R is only rotated.  The bf16 path also folds alpha^q into q~.
#include "device_common.h"
#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {

// cos/sin of the query position for every RoPE pair, into LDS (cs[2*i],
// cs[2*i+1]).
__device__ void rope_table(int pos, int dr, float base, float* cs) {
  for (int i = threadIdx.x; i < dr / 2; i += blockDim.x) rope_cos_sin(pos, i, dr, base, &cs[2 * i], &cs[2 * i + 1]);
}

// alpha^q and the RoPE query of one head; executed by one wavefront
// (lane-strided over dims).  cs: the rope_table of the query position.
template <typename TIn, typename TOut>
__device__ void prep_scalar_and_rope(const TIn* qc, const TIn* qr, const float* gqr, int dc,
                                     int dr, float eps, float tau, int qk_norm, const float* cs,
                                     float* alpha_q_out, TOut* qr_out) {
  const int lane = threadIdx.x & 63;
  const float sl = tau * kLog2e;
  float ss = 0.f;
  if (qk_norm) {
    for (int e = lane; e < dc; e += 64) {
      float v = Elem<TIn>::load(qc, e);
      ss += v * v;
    }
    ss = wave_sum(ss);
  }
  float aq = qk_norm ? 1.0f / sqrtf(ss / (float)dc + eps) : 1.0f;
  if (lane == 0) *alpha_q_out = aq * sl;
  float rs = 0.f;
  if (qk_norm) {
    for (int e = lane; e < dr; e += 64) {
      float v = Elem<TIn>::load(qr, e);
      rs += v * v;
    }
    rs = wave_sum(rs);
  }
  float rscale = qk_norm ? 1.0f / sqrtf(rs / (float)dr + eps) : 1.0f;
  for (int pi = lane; pi < dr / 2; pi += 64) {
    float x0 = Elem<TIn>::load(qr, 2 * pi), x1 = Elem<TIn>::load(qr, 2 * pi + 1);
    if (qk_norm) {
      x0 *= rscale * gqr[2 * pi];
      x1 *= rscale * gqr[2 * pi + 1];
    }
    const float c = cs[2 * pi], sn = cs[2 * pi + 1];
    Elem<TOut>::store(qr_out, 2 * pi, (x0 * c - x1 * sn) * sl);
    Elem<TOut>::store(qr_out, 2 * pi + 1, (x0 * sn + x1 * c) * sl);
  }
}

// Paged caches: every block-table entry the sequence's rows need must name a
// page of the pool; otherwise QKMLA_DEV_BAD_PAGE (the decode then reads page 0
// in its place, and that sequence's output is undefined).  Checked once per
// sequence, by its last query row (the longest prefix); block-wide.
__device__ void check_pages(const Paging& pg, int v, int s_q, int L, int32_t* status) {
  if (!pg.bt || !status || v % s_q != s_q - 1 || L < 1 || L > pg.capacity()) return;
  const int nblk = (L + pg.page_size - 1) / pg.page_size;
  bool bad = false;
  for (int blk = threadIdx.x; blk < nblk; blk += blockDim.x) bad |= pg.page_of(v / s_q, blk) < 0;
  if (bad) atomicOr(status, QKMLA_DEV_BAD_PAGE);
}

__device__ __forceinline__ int clamp_pos(int L, int L_cap) {
  return (L >= 1 && L <= L_cap) ? L - 1 : 0;
}

// bf16 layer with 16 heads per KV group: one workgroup (4 waves) per (b, g).
// q~[16 heads][r] = q^C[16][d_c] . W~_g^T[d_c][r] on mfma_f32_16x16x32_bf16.
// Operand layouts (gfx950, 16x16x32): A lane l holds A[m=l%16][k=8(l/16)+j],
// B lane l holds B[k=8(l/16)+j][n=l%16], D lane l reg i holds D[4(l/16)+i][l%16].
__global__ __launch_bounds__(256) void qprep_mfma_kernel(
    const uint16_t* __restrict__ q_c, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_qabs, const float* __restrict__ gqr,
    const int32_t* __restrict__ seq_lens, int s_q, const Paging pg, int H, int G, int r, int dc,
    int dr, float eps, float tau, float base, int qk_norm, uint16_t* __restrict__ q_tilde,
    float* __restrict__ alpha_q, uint16_t* __restrict__ q_rope_out, int32_t* status) {
  const int b = blockIdx.x, g = blockIdx.y;  // b: virtual sequence (query row)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h0 = g * 16;
  const int L_cap = pg.capacity();
  const int L = virt_len(seq_lens, b, s_q, L_cap);
  if (g == 0) check_pages(pg, b, s_q, L, status);
  if (g == 0 && threadIdx.x == 0 && (L < 1 || L > L_cap) && status)
    atomicOr(status, QKMLA_DEV_BAD_SEQ_LEN);
  const int pos = clamp_pos(L, L_cap);

  __shared__ float cs[256];  // d_r <= 256
  rope_table(pos, dr, base, cs);

  const uint16_t* A = q_c + ((size_t)b * H + h0) * dc;
  const uint16_t* W = w_qabs + (size_t)g * r * dc;
  const int m = lane & 15, kq = lane >> 4;
  // Per-head scale folded into q~: the decode logit is then one FMA,
  // S_c * alpha^k + S_r, with alpha^q, the softmax scale and log2(e) already
  // in q~ (QK-norm); plain mode has one accumulator for content + RoPE, so
  // only the softmax scale and log2(e) go in.
  __shared__ float qscale[16];
  for (int hh = wave; hh < 16; hh += 4) {
    const uint16_t* qh = A + (size_t)hh * dc;
    float ss = 0.f;
    for (int e = lane; e < dc; e += 64) {
      const float v = bf16_to_f32(qh[e]);
      ss += v * v;
    }
    ss = wave_sum(ss);
    if (lane == 0)
      qscale[hh] = (qk_norm ? 1.0f / sqrtf(ss / (float)dc + eps) : 1.0f) * (tau * kLog2e);
  }
  __syncthreads();
  // The bf16 path has r = 512: each wave owns 8 blocks of 16 output columns.
  // The loops are unrolled so that every weight load is issued before the
  // first MFMA waits (the weights come from L2 or HBM, one latency, not eight).
  constexpr int kNbPerWave = 512 / 16 / 4;
  const int ksteps = dc / 32;               // 4 for d_c = 128
  constexpr int kMaxK = 8;                  // d_c <= 256 on this path
  bf16x8 a[kMaxK];
#pragma unroll
  for (int ks = 0; ks < kMaxK; ++ks)
    if (ks < ksteps) a[ks] = *(const bf16x8*)(A + (size_t)m * dc + ks * 32 + kq * 8);
  f32x4 acc[kNbPerWave];
#pragma unroll
  for (int nbi = 0; nbi < kNbPerWave; ++nbi) acc[nbi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kMaxK; ++ks) {
    if (ks < ksteps) {
      bf16x8 bv[kNbPerWave];
#pragma unroll
      for (int nbi = 0; nbi < kNbPerWave; ++nbi)
        bv[nbi] = *(const bf16x8*)(W + (size_t)((wave * kNbPerWave + nbi) * 16 + m) * dc +
                                   kq * 8 + ks * 32);
#pragma unroll
      for (int nbi = 0; nbi < kNbPerWave; ++nbi)
        acc[nbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bv[nbi], acc[nbi], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nbi = 0; nbi < kNbPerWave; ++nbi) {
    const int nb = wave * kNbPerWave + nbi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int hh = 4 * kq + i;
      q_tilde[((size_t)b * H + h0 + hh) * r + nb * 16 + m] = f32_to_bf16(acc[nbi][i] * qscale[hh]);
    }
  }
  __syncthreads();  // cs ready
  // alpha^q and the RoPE query: each wave takes 4 of the 16 heads.
  for (int hh = wave; hh < 16; hh += 4) {
    int h = h0 + hh;
    prep_scalar_and_rope<uint16_t, uint16_t>(
        q_c + ((size_t)b * H + h) * dc, q_rope + ((size_t)b * H + h) * dr, gqr, dc, dr, eps, tau,
        qk_norm, cs, alpha_q + (size_t)b * H + h, q_rope_out + ((size_t)b * H + h) * dr);
  }
}

// Any shape, float storage: one workgroup per (b, h).
__global__ __launch_bounds__(256) void qprep_generic_kernel(
    const float* __restrict__ q_c, const float* __restrict__ q_rope,
    const float* __restrict__ w_qabs, const float* __restrict__ gqr,
    const int32_t* __restrict__ seq_lens, int s_q, const Paging pg, int H, int G, int r, int dc,
    int dr, float eps, float tau, float base, int qk_norm, float* __restrict__ q_tilde,
    float* __restrict__ alpha_q, float* __restrict__ q_rope_out, int32_t* status) {
  const int b = blockIdx.x, h = blockIdx.y;  // b: virtual sequence (query row)
  const int g = (h * G) / H;
  const int L_cap = pg.capacity();
  const int L = virt_len(seq_lens, b, s_q, L_cap);
  if (h == 0) check_pages(pg, b, s_q, L, status);
  if (h == 0 && threadIdx.x == 0 && (L < 1 || L > L_cap) && status)
    atomicOr(status, QKMLA_DEV_BAD_SEQ_LEN);
  const int pos = clamp_pos(L, L_cap);
  const float* qc = q_c + ((size_t)b * H + h) * dc;
  const float* W = w_qabs + (size_t)g * r * dc;
  for (int i = threadIdx.x; i < r; i += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < dc; ++j) acc += qc[j] * W[(size_t)i * dc + j];
    q_tilde[((size_t)b * H + h) * r + i] = acc;
  }
  __shared__ float cs[256];  // d_r <= 256
  rope_table(pos, dr, base, cs);
  __syncthreads();
  if (threadIdx.x < 64)
    prep_scalar_and_rope<float, float>(qc, q_rope + ((size_t)b * H + h) * dr, gqr, dc, dr, eps,
                                       tau, qk_norm, cs, alpha_q + (size_t)b * H + h,
                                       q_rope_out + ((size_t)b * H + h) * dr);
}

hipError_t launch_qprep(const Cfg& c, int batch, int s_q, const void* q_c, const void* q_rope,
                        const void* w_qabs, const float* gqr, const int32_t* seq_lens,
                        const Paging& pg, const WsLayout& ws, void* workspace, int32_t* status,
                        hipStream_t s) {
  char* wsb = (char*)workspace;
  const int nv = batch * s_q;  // virtual sequences, one per query row
  if (c.dtype == QKMLA_BF16) {
    qprep_mfma_kernel<<<dim3(nv, c.G), 256, 0, s>>>(
        (const uint16_t*)q_c, (const uint16_t*)q_rope, (const uint16_t*)w_qabs, gqr, seq_lens,
        s_q, pg, c.H, c.G, c.r, c.dc, c.dr, c.eps, c.tau, c.base, c.qk_norm,
        (uint16_t*)(wsb + ws.q_tilde), (float*)(wsb + ws.alpha_q), (uint16_t*)(wsb + ws.q_rope),
        status);
  } else {
    qprep_generic_kernel<<<dim3(nv, c.H), 256, 0, s>>>(
        (const float*)q_c, (const float*)q_rope, (const float*)w_qabs, gqr, seq_lens, s_q, pg, c.H,
        c.G, c.r, c.dc, c.dr, c.eps, c.tau, c.base, c.qk_norm, (float*)(wsb + ws.q_tilde),
        (float*)(wsb + ws.alpha_q), (float*)(wsb + ws.q_rope), status);
  }
  return hipGetLastError();
}

}  // namespace qkmla
