// Decode for float storage and arbitrary (small) layer shapes: one workgroup
// per (sequence, head) streams the whole sequence with an exact online
// softmax over chunks of 256 tokens.  Same mathematics as the MFMA kernel:
//   logit_t = (q~_h . c_t) alpha^q_h alpha^k_{t,g} + q^R_h . k^R_t   (exp2 domain)
// ("QK-Normed MLA: QK normalization without full key caching", technical
// summary, Methodology: decode-logit formula and row-column scaling).
#include "device_common.h"
#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {

constexpr int kGenChunk = 256;
constexpr int kGenMaxR = 1024;
constexpr int kGenMaxDr = 256;

__global__ __launch_bounds__(256) void decode_generic_kernel(
    const int32_t* __restrict__ seq_lens, int s_q, Paging pg, int H, int G, int r, int dr, int qk_norm,
    const float* __restrict__ lat, const float* __restrict__ rope, const float* __restrict__ alpha,
    const float* __restrict__ q_tilde, const float* __restrict__ alpha_q,
    const float* __restrict__ q_rope, float* __restrict__ o_lat, float* __restrict__ lse) {
  __shared__ float qt[kGenMaxR];
  __shared__ float qr[kGenMaxDr];
  __shared__ float p[kGenChunk];
  __shared__ int64_t prow[kGenChunk];  // physical cache row of each token of the chunk
  __shared__ float red[4];
  // b: virtual sequence (query row b % s_q of cache b / s_q)
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int bc = b / s_q;
  const int g = (h * G) / H;
  const int L_cap = pg.capacity();
  const int L = virt_len(seq_lens, b, s_q, L_cap);
  float* out = o_lat + ((size_t)b * H + h) * r;
  if (L < 1 || L > L_cap) {
    for (int i = tid; i < r; i += blockDim.x) out[i] = 0.f;
    if (tid == 0 && lse) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  for (int i = tid; i < r; i += blockDim.x) qt[i] = q_tilde[((size_t)b * H + h) * r + i];
  for (int i = tid; i < dr; i += blockDim.x) qr[i] = q_rope[((size_t)b * H + h) * dr + i];
  const float aq = alpha_q[(size_t)b * H + h];
  __syncthreads();
  // each thread owns output dims tid, tid+256, ... (r <= 1024 -> 4 per thread)
  float acc[kGenMaxR / 256];
#pragma unroll
  for (int k = 0; k < kGenMaxR / 256; ++k) acc[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int t0 = 0; t0 < L; t0 += kGenChunk) {
    const int t = t0 + tid;
    float logit = -INFINITY;
    if (t < L) {
      // a block-table entry outside the pool reads page 0 (q-prep reports it)
      const int64_t pr = pg.phys_row(bc, t);
      const int64_t row = pr < 0 ? (int64_t)(t % pg.page_size) : pr;
      prow[tid] = row;
      const float* c = lat + (size_t)row * r;
      float sc = 0.f;
      for (int i = 0; i < r; ++i) sc += qt[i] * c[i];
      const float* kr = rope + (size_t)row * dr;
      float sr = 0.f;
      for (int i = 0; i < dr; ++i) sr += qr[i] * kr[i];
      float ak = qk_norm ? alpha[(size_t)row * G + g] : 1.0f;
      logit = sc * (aq * ak) + sr;
    }
    // chunk max
    float mx = logit;
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    float m_chunk = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float m_new = fmaxf(m_run, m_chunk);
    float f = exp2f(m_run - m_new);  // 0 on the first chunk
    float pv = (t < L) ? exp2f(logit - m_new) : 0.f;
    p[tid] = pv;
    float s = wave_sum(pv);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    l_run = l_run * f + (red[0] + red[1] + red[2] + red[3]);
    m_run = m_new;
    const int n = min(kGenChunk, L - t0);
#pragma unroll
    for (int k = 0; k < kGenMaxR / 256; ++k) {
      int i = tid + 256 * k;
      if (i < r) {
        float a = acc[k] * f;
        for (int tt = 0; tt < n; ++tt) a += p[tt] * lat[(size_t)prow[tt] * r + i];
        acc[k] = a;
      }
    }
    __syncthreads();
  }
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int k = 0; k < kGenMaxR / 256; ++k) {
    int i = tid + 256 * k;
    if (i < r) out[i] = acc[k] * inv;
  }
  if (tid == 0 && lse) lse[(size_t)b * H + h] = (m_run + log2f(l_run)) * kLn2;
}

hipError_t launch_decode_generic(const Cfg& c, int batch, int s_q, const int32_t* seq_lens,
                                 const Paging& pg, const void* lat, const void* rope,
                                 const float* alpha,
                                 const WsLayout& ws, void* workspace, float* o_lat, float* lse,
                                 hipStream_t s) {
  char* wsb = (char*)workspace;
  return launch_kernel(decode_generic_kernel, dim3(batch * s_q, c.H), dim3(256), s, seq_lens, s_q,
                       pg, c.H, c.G, c.r, c.dr, c.qk_norm, (const float*)lat, (const float*)rope,
                       alpha, (const float*)(wsb + ws.q_tilde), (const float*)(wsb + ws.alpha_q),
                       (const float*)(wsb + ws.q_rope), o_lat, lse);
}

}  // namespace qkmla
