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
#include <cmath>

#include "device_common.h"
#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {

RopeFreq rope_freq(int dr, float base) {
  RopeFreq rf;
  for (int i = 0; i < kMaxRopePairs; ++i)
    rf.f[i] = i < dr / 2 ? std::pow((double)base, -2.0 * (double)i / (double)dr) : 0.0;
  return rf;
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

// Sequence-level status bits (length outside [1, L_cap], bad pages); called
// by one block per virtual sequence, block-wide.
__device__ void check_sequence(const Paging& pg, int v, int s_q, int L, int32_t* status) {
  check_pages(pg, v, s_q, L, status);
  if (threadIdx.x == 0 && (L < 1 || L > pg.capacity()) && status)
    atomicOr(status, QKMLA_DEV_BAD_SEQ_LEN);
}

// bf16 layer with 16 heads per KV group.  For group g the query projection
// is a GEMM  q~[(sequence, head)][r] = q^C[(sequence, head)][d_c] . W~_g^T
// (mfma_f32_16x16x32_bf16, fp32 accumulation).  Grid (ceil(nv / SPB), G,
// r / kQpCols + 1), 256 threads: block (x, g, z < r / kQpCols) takes the
// group's 16 heads of SPB sequences (M = 16 SPB rows) and output columns
// [z kQpCols, (z+1) kQpCols); wave w owns two 16-wide column blocks at
// z kQpCols + 32 w for all M rows, so each W~ element the block needs is
// loaded once and serves SPB sequences.  Every operand load is issued before
// the first MFMA.  Each lane also holds a quarter of its row's q^C (the A
// operand), so alpha^q comes from the same registers with two cross-lane
// sums.  The tile goes out through LDS as 16-byte stores.  The last z-slice
// writes the normalised, rotated RoPE query of the block's rows and the
// sequences' status bits, its loads likewise issued together.
// Layouts (gfx950, 16x16x32): A lane l holds A[m=l%16][k=8(l/16)+j], B lane l
// holds B[k=8(l/16)+j][n=l%16], D lane l reg i holds D[4(l/16)+i][l%16].
constexpr int kQpCols = 128;
constexpr int kQpRopeSlots = 4;  // RoPE pairs per thread and sequence: 16 threads per head, d_r / 2 <= 64

template <int SPB, int KS>
__global__ __launch_bounds__(256) void qprep_mfma_kernel(
    const uint16_t* __restrict__ q_c, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_qabs, const float* __restrict__ gqr,
    const int32_t* __restrict__ seq_lens, int nv, int s_q, const Paging pg, int H, int r, int dr,
    float eps, float tau, int qk_norm, const RopeFreq rf, uint16_t* __restrict__ q_tilde,
    float* __restrict__ alpha_q, uint16_t* __restrict__ q_rope_out, int32_t* status) {
  constexpr int dc = KS * 32;
  const int b0 = blockIdx.x * SPB, g = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h0 = g * 16;
  const float sl = tau * kLog2e;

  if (z == r / kQpCols) {
    // ---- RoPE query: thread -> head hh of each sequence, pairs p0, p0 + 16, ... ----
    const int hh = tid >> 4, p0 = tid & 15;
    const int np = dr / 2;
    const int L_cap = pg.capacity();
    uint32_t u[SPB][kQpRopeSlots];
    float2 gg[kQpRopeSlots];
    double fr[kQpRopeSlots];
    int L[SPB];
#pragma unroll
    for (int k = 0; k < kQpRopeSlots; ++k) {
      const int pi = min(p0 + 16 * k, np - 1);  // pairs past d_r / 2 re-read the last one
      gg[k] = *(const float2*)(gqr + 2 * pi);
      fr[k] = rf.f[pi];
#pragma unroll
      for (int sq = 0; sq < SPB; ++sq) {
        const int b = min(b0 + sq, nv - 1);
        u[sq][k] = *(const uint32_t*)(q_rope + ((size_t)b * H + h0 + hh) * dr + 2 * pi);
      }
    }
#pragma unroll
    for (int sq = 0; sq < SPB; ++sq) L[sq] = virt_len(seq_lens, min(b0 + sq, nv - 1), s_q, L_cap);
#pragma unroll
    for (int sq = 0; sq < SPB; ++sq) {
      const int b = b0 + sq;
      float rs = 0.f;
#pragma unroll
      for (int k = 0; k < kQpRopeSlots; ++k) {
        const float x0 = bf16_to_f32((uint16_t)u[sq][k]), x1 = bf16_to_f32((uint16_t)(u[sq][k] >> 16));
        rs += p0 + 16 * k < np ? x0 * x0 + x1 * x1 : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rs += __shfl_xor(rs, o, 64);
      const float rscale = qk_norm ? 1.0f / sqrtf(rs / (float)dr + eps) : 1.0f;
      const int pos = clamp_pos(L[sq], L_cap);
#pragma unroll
      for (int k = 0; k < kQpRopeSlots; ++k) {
        const int pi = p0 + 16 * k;
        if (pi < np && b < nv) {
          float x0 = bf16_to_f32((uint16_t)u[sq][k]), x1 = bf16_to_f32((uint16_t)(u[sq][k] >> 16));
          if (qk_norm) {
            x0 *= rscale * gg[k].x;
            x1 *= rscale * gg[k].y;
          }
          float c, sn;
          rope_cos_sin_freq(pos, fr[k], &c, &sn);
          *(uint32_t*)(q_rope_out + qop_index(b, H, dr, h0 + hh, 2 * pi)) =
              (uint32_t)f32_to_bf16((x0 * c - x1 * sn) * sl) |
              ((uint32_t)f32_to_bf16((x0 * sn + x1 * c) * sl) << 16);
        }
      }
    }
    if (g == 0)
      for (int sq = 0; sq < SPB; ++sq)
        if (b0 + sq < nv) check_sequence(pg, b0 + sq, s_q, L[sq], status);
    return;
  }

  // ---- q~ columns [z kQpCols, (z+1) kQpCols) of SPB sequences ----
  // (rows padded by 16 bytes: the column-wise reads below hit distinct banks)
  __shared__ __attribute__((aligned(16))) uint16_t tile[16 * SPB][kQpCols + 8];
  const int m = lane & 15, kq = lane >> 4;
  const uint16_t* W = w_qabs + (size_t)g * r * dc;
  const int n0 = z * kQpCols + wave * 32;
  bf16x8 a[SPB][KS], bv[2][KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      bv[nb][ks] = *(const bf16x8*)(W + (size_t)(n0 + nb * 16 + m) * dc + ks * 32 + kq * 8);
#pragma unroll
    for (int sq = 0; sq < SPB; ++sq) {
      const int b = min(b0 + sq, nv - 1);  // rows past the batch repeat its last one, unstored
      a[sq][ks] = *(const bf16x8*)(q_c + ((size_t)b * H + h0 + m) * dc + ks * 32 + kq * 8);
    }
  }
  f32x4 acc[SPB][2];
  float aq[SPB];
#pragma unroll
  for (int sq = 0; sq < SPB; ++sq) {
    // alpha^q of row m (lanes m, m+16, m+32, m+48 hold a quarter of q^C each),
    // times the softmax scale and log2(e)
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = (float)a[sq][ks][j];
        ss += v * v;
      }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    aq[sq] = (qk_norm ? 1.0f / sqrtf(ss / (float)dc + eps) : 1.0f) * sl;
    if (z == 0 && wave == 0 && kq == 0 && b0 + sq < nv) alpha_q[(size_t)(b0 + sq) * H + h0 + m] = aq[sq];
    acc[sq][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[sq][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int sq = 0; sq < SPB; ++sq)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[sq][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sq][ks], bv[nb][ks], acc[sq][nb], 0, 0, 0);
#pragma unroll
  for (int sq = 0; sq < SPB; ++sq)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * kq + i;
      const float sc = __shfl(aq[sq], hh, 64);  // lane hh (< 16) holds row hh's scale
      tile[16 * sq + hh][wave * 32 + m] = f32_to_bf16(acc[sq][0][i] * sc);
      tile[16 * sq + hh][wave * 32 + 16 + m] = f32_to_bf16(acc[sq][1][i] * sc);
    }
  __syncthreads();
  // 16 SPB rows x 128 columns of bf16, 16 bytes per thread and step; the 16
  // threads of a group take the 16 heads of one 8-column chunk, which lie
  // contiguous in the operand order (256 bytes per group).
#pragma unroll
  for (int it = 0; it < SPB; ++it) {
    const int row = it * 16 + (tid & 15), c8 = (tid >> 4) * 8;
    const int b = b0 + it;
    if (b < nv)
      *(uint4*)(q_tilde + qop_index(b, H, r, h0 + (tid & 15), z * kQpCols + c8)) =
          *(const uint4*)&tile[row][c8];
  }
}

template <int SPB, int KS>
static hipError_t launch_qprep_bf16(const Cfg& c, int nv, int s_q, const void* q_c, const void* q_rope,
                              const void* w_qabs, const float* gqr, const int32_t* seq_lens,
                              const Paging& pg, const RopeFreq& rf, char* wsb, const WsLayout& ws,
                              int32_t* status, hipStream_t s) {
  return launch_kernel(qprep_mfma_kernel<SPB, KS>,
                       dim3((nv + SPB - 1) / SPB, c.G, c.r / kQpCols + 1), dim3(256), s, (const uint16_t*)q_c, (const uint16_t*)q_rope,
                (const uint16_t*)w_qabs, gqr, seq_lens, nv, s_q, pg, c.H, c.r, c.dr, c.eps, c.tau,
                c.qk_norm, rf, (uint16_t*)(wsb + ws.q_tilde), (float*)(wsb + ws.alpha_q),
                (uint16_t*)(wsb + ws.q_rope), status);
}

template <int SPB>
static hipError_t launch_qprep_spb(const Cfg& c, int nv, int s_q, const void* q_c, const void* q_rope,
                             const void* w_qabs, const float* gqr, const int32_t* seq_lens,
                             const Paging& pg, const RopeFreq& rf, char* wsb, const WsLayout& ws,
                             int32_t* status, hipStream_t s) {
#define QP_CASE(K)                                                                           \
  case K:                                                                                    \
    return launch_qprep_bf16<SPB, K>(c, nv, s_q, q_c, q_rope, w_qabs, gqr, seq_lens, pg, rf, \
                                     wsb, ws, status, s);
  switch (c.dc / 32) {
    QP_CASE(1) QP_CASE(2) QP_CASE(3) QP_CASE(4) QP_CASE(5) QP_CASE(6) QP_CASE(7) QP_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef QP_CASE
}

// Any shape, float storage: one workgroup per (b, h).
__global__ __launch_bounds__(256) void qprep_generic_kernel(
    const float* __restrict__ q_c, const float* __restrict__ q_rope,
    const float* __restrict__ w_qabs, const float* __restrict__ gqr,
    const int32_t* __restrict__ seq_lens, int s_q, const Paging pg, int H, int G, int r, int dc,
    int dr, float eps, float tau, int qk_norm, const RopeFreq rf, float* __restrict__ q_tilde,
    float* __restrict__ alpha_q, float* __restrict__ q_rope_out, int32_t* status) {
  const int b = blockIdx.x, h = blockIdx.y;  // b: virtual sequence (query row)
  const int g = (h * G) / H;
  const int L_cap = pg.capacity();
  const int L = virt_len(seq_lens, b, s_q, L_cap);
  if (h == 0) check_sequence(pg, b, s_q, L, status);
  const int pos = clamp_pos(L, L_cap);
  const float* qc = q_c + ((size_t)b * H + h) * dc;
  const float* W = w_qabs + (size_t)g * r * dc;
  for (int i = threadIdx.x; i < r; i += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < dc; ++j) acc += qc[j] * W[(size_t)i * dc + j];
    q_tilde[((size_t)b * H + h) * r + i] = acc;
  }
  if (threadIdx.x >= 64) return;
  // alpha^q and the RoPE query, one wavefront (lane-strided over dims)
  const int lane = threadIdx.x;
  const float sl = tau * kLog2e;
  const float* qr = q_rope + ((size_t)b * H + h) * dr;
  float ss = 0.f, rs = 0.f;
  if (qk_norm) {
    for (int e = lane; e < dc; e += 64) ss += qc[e] * qc[e];
    for (int e = lane; e < dr; e += 64) rs += qr[e] * qr[e];
    ss = wave_sum(ss);
    rs = wave_sum(rs);
  }
  const float aq = qk_norm ? 1.0f / sqrtf(ss / (float)dc + eps) : 1.0f;
  if (lane == 0) alpha_q[(size_t)b * H + h] = aq * sl;
  const float rscale = qk_norm ? 1.0f / sqrtf(rs / (float)dr + eps) : 1.0f;
  float* qo = q_rope_out + ((size_t)b * H + h) * dr;
  for (int pi = lane; pi < dr / 2; pi += 64) {
    float x0 = qr[2 * pi], x1 = qr[2 * pi + 1];
    if (qk_norm) {
      x0 *= rscale * gqr[2 * pi];
      x1 *= rscale * gqr[2 * pi + 1];
    }
    float c, sn;
    rope_cos_sin_freq(pos, rf.f[pi], &c, &sn);
    qo[2 * pi] = (x0 * c - x1 * sn) * sl;
    qo[2 * pi + 1] = (x0 * sn + x1 * c) * sl;
  }
}

hipError_t launch_qprep(const Cfg& c, int batch, int s_q, const void* q_c, const void* q_rope,
                        const void* w_qabs, const float* gqr, const int32_t* seq_lens,
                        const Paging& pg, const WsLayout& ws, void* workspace, int32_t* status,
                        hipStream_t s) {
  char* wsb = (char*)workspace;
  const int nv = batch * s_q;  // virtual sequences, one per query row
  const RopeFreq rf = rope_freq(c.dr, c.base);
  if (c.dtype == QKMLA_BF16) {
    // Two sequences share a block's W~ loads once the batch gives enough
    // blocks (measured on the 128-head layer: at 16 and 64 sequences two per
    // block beat one and four).
    if (nv >= 16)
      return launch_qprep_spb<2>(c, nv, s_q, q_c, q_rope, w_qabs, gqr, seq_lens, pg, rf, wsb, ws,
                                 status, s);
    return launch_qprep_spb<1>(c, nv, s_q, q_c, q_rope, w_qabs, gqr, seq_lens, pg, rf, wsb, ws,
                               status, s);
  } else {
    return launch_kernel(qprep_generic_kernel, dim3(nv, c.H), dim3(256), s, (const float*)q_c,
                  (const float*)q_rope, (const float*)w_qabs, gqr, seq_lens, s_q, pg, c.H, c.G,
                  c.r, c.dc, c.dr, c.eps, c.tau, c.qk_norm, rf, (float*)(wsb + ws.q_tilde),
                  (float*)(wsb + ws.alpha_q), (float*)(wsb + ws.q_rope), status);
  }
}

}  // namespace qkmla
