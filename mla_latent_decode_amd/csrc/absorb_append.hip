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
    const int32_t* __restrict__ positions, int L_cap, T* __restrict__ lat, T* __restrict__ rope,
    float* __restrict__ alpha, int32_t* status, int G, int r, int dc, int dr, float eps,
    float base, int qk_norm) {
  __shared__ float cs[kAppendTok * kMaxR];
  __shared__ float ksq[kAppendTok];
  __shared__ float rsum[kAppendTok];
  const int T_total = batch * n_new;
  const int tok0 = blockIdx.x * kAppendTok;
  const int duty = blockIdx.y;
  const bool copy_duty = qk_norm ? (duty == G) : (duty == 0);
  const int tid = threadIdx.x;

  if (copy_duty) {
    for (int k = 0; k < kAppendTok; ++k) {
      int tok = tok0 + k;
      if (tok >= T_total) break;
      int b = tok / n_new, i = tok % n_new;
      int pos0 = positions[b];
      bool bad = pos0 < 0 || (int64_t)pos0 + n_new > L_cap;
      if (bad) {
        if (tid == 0 && i == 0 && status) atomicOr(status, QKMLA_DEV_BAD_POSITION);
        continue;
      }
      int row = pos0 + i;
      const T* src = c_new + (size_t)tok * r;
      T* dst = lat + ((size_t)b * L_cap + row) * r;
      for (int e = tid; e < r; e += blockDim.x) dst[e] = src[e];
      // RoPE key: optional RMSNorm over d_r, then rotate pairs by row position.
      const T* ks = kr_new + (size_t)tok * dr;
      float scale = 1.f;
      if (qk_norm) {
        if (tid < 64) {
          float acc = 0.f;
          for (int e = tid; e < dr; e += 64) {
            float v = Elem<T>::load(ks, e);
            acc += v * v;
          }
          acc = wave_sum(acc);
          if (tid == 0) rsum[k] = acc;
        }
        __syncthreads();
        scale = 1.0f / sqrtf(rsum[k] / (float)dr + eps);
      }
      T* rdst = rope + ((size_t)b * L_cap + row) * dr;
      for (int pi = tid; pi < dr / 2; pi += blockDim.x) {
        float x0 = Elem<T>::load(ks, 2 * pi), x1 = Elem<T>::load(ks, 2 * pi + 1);
        if (qk_norm) {
          x0 = x0 * scale * gkr[2 * pi];
          x1 = x1 * scale * gkr[2 * pi + 1];
        }
        float cs_, sn_;
        rope_cos_sin(row, pi, dr, base, &cs_, &sn_);
        Elem<T>::store(rdst, 2 * pi, x0 * cs_ - x1 * sn_);
        Elem<T>::store(rdst, 2 * pi + 1, x0 * sn_ + x1 * cs_);
      }
      __syncthreads();
    }
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
    bool bad = pos0 < 0 || (int64_t)pos0 + n_new > L_cap;
    if (!bad) {
      float a = 1.0f / sqrtf(ksq[tid] / (float)dc + eps);
      alpha[((size_t)b * L_cap + pos0 + i) * G + g] = a;
    }
  }
}

hipError_t launch_append(const Cfg& c, int batch, int n_new, const void* c_new,
                         const void* k_rope_new, const float* w_uk, const float* gkr,
                         const int32_t* positions, int L_cap, void* lat, void* rope, float* alpha,
                         int32_t* status, hipStream_t s) {
  int T_total = batch * n_new;
  dim3 grid((unsigned)((T_total + kAppendTok - 1) / kAppendTok), c.qk_norm ? c.G + 1 : 1);
  if (c.dtype == QKMLA_BF16)
    append_kernel<uint16_t><<<grid, 256, 0, s>>>(
        batch, n_new, (const uint16_t*)c_new, (const uint16_t*)k_rope_new, w_uk, gkr, positions,
        L_cap, (uint16_t*)lat, (uint16_t*)rope, alpha, status, c.G, c.r, c.dc, c.dr, c.eps,
        c.base, c.qk_norm);
  else
    append_kernel<float><<<grid, 256, 0, s>>>(
        batch, n_new, (const float*)c_new, (const float*)k_rope_new, w_uk, gkr, positions, L_cap,
        (float*)lat, (float*)rope, alpha, status, c.G, c.r, c.dc, c.dr, c.eps, c.base,
        c.qk_norm);
  return hipGetLastError();
}

}  // namespace qkmla
