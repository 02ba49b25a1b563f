// Split merge and V up-projection.
//
// merge: the log-sum-exp combination of split-KV partials of one sequence
//   (exp2 domain):  M = max_s m_s,  w_s = 2^(m_s - M),
//   o_lat = sum_s w_s O_s / sum_s w_s l_s,  lse = (M + log2 sum_s w_s l_s) ln 2.
// out_proj: o[b][h][:] = o_lat[b][h][:] W^UV_{g(h)} -- the value side of MLA,
//   linear in the latent ("QK-Normed MLA: QK normalization without full key
//   caching", technical summary, Problem Statement: the latent state stands in
//   for keys and values and is up-projected at decode).
#include "device_common.h"
#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {

// grid (B, H/4), 256 threads: 4 heads per block, 64 threads per head, r/64
// dims per thread (r = 512 -> 8).
__global__ __launch_bounds__(256) void merge_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                    int L_cap, int H, int r, int n_wg,
                                                    const float* __restrict__ part,
                                                    float* __restrict__ o_lat,
                                                    float* __restrict__ lse) {
  __shared__ int P[kMaxBatch + 1];
  build_tile_prefix(seq_lens, B, L_cap, P);
  const int b = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int dpt = r / 64;
  float* out = o_lat + ((size_t)b * H + h) * r + lane * dpt;
  const int n_b = P[b + 1] - P[b];
  if (n_b == 0) {  // invalid length: zeros and lse = -inf
    for (int i = 0; i < dpt; ++i) out[i] = 0.f;
    if (lane == 0 && lse) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const int64_t N = P[B];
  const int p_lo = wg_of(P[b], N, n_wg);
  const int p_hi = wg_of(P[b + 1] - 1, N, n_wg);
  if (p_lo == p_hi) return;  // written directly by the decode kernel
  const size_t slot_floats = (size_t)H * (r + 2);
  const int slot_lo = (wg_start(p_lo, N, n_wg) == P[b]) ? 0 : 1;
  // Workgroups between p_lo and p_hi with an empty range (more workgroups
  // than tiles) wrote nothing and are skipped.
  float M = -INFINITY;
  for (int p = p_lo; p <= p_hi; ++p) {
    if (p != p_lo && wg_start(p, N, n_wg) == wg_start(p + 1, N, n_wg)) continue;
    const float* s = part + ((size_t)p * kSlotsPerWg + (p == p_lo ? slot_lo : 0)) * slot_floats;
    M = fmaxf(M, s[h]);
  }
  float acc[16];
  for (int i = 0; i < dpt; ++i) acc[i] = 0.f;
  float lsum = 0.f;
  for (int p = p_lo; p <= p_hi; ++p) {
    if (p != p_lo && wg_start(p, N, n_wg) == wg_start(p + 1, N, n_wg)) continue;
    const float* s = part + ((size_t)p * kSlotsPerWg + (p == p_lo ? slot_lo : 0)) * slot_floats;
    float w = exp2f(s[h] - M);
    lsum += w * s[H + h];
    const float* O = s + 2 * H + (size_t)h * r + lane * dpt;
    for (int i = 0; i < dpt; i += 4) {
      f32x4 v = *(const f32x4*)(O + i);
      acc[i] += w * v[0];
      acc[i + 1] += w * v[1];
      acc[i + 2] += w * v[2];
      acc[i + 3] += w * v[3];
    }
  }
  const float inv = 1.0f / lsum;
  for (int i = 0; i < dpt; i += 4) {
    f32x4 v = {acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
    *(f32x4*)(out + i) = v;
  }
  if (lane == 0 && lse) lse[(size_t)b * H + h] = (M + log2f(lsum)) * kLn2;
}

hipError_t launch_merge(const Cfg& c, int batch, const int32_t* seq_lens, int L_cap,
                        const WsLayout& ws, void* workspace, int n_wg, float* o_lat, float* lse,
                        hipStream_t s) {
  char* wsb = (char*)workspace;
  merge_kernel<<<dim3(batch, c.H / 4), 256, 0, s>>>(seq_lens, batch, L_cap, c.H, c.r, n_wg,
                                                     (const float*)(wsb + ws.partials), o_lat,
                                                     lse);
  return hipGetLastError();
}

// One block per (b, h); threads over the d_v outputs.
template <typename T>
__global__ __launch_bounds__(256) void out_proj_kernel(const float* __restrict__ o_lat,
                                                       const T* __restrict__ w_uv,
                                                       float* __restrict__ out, int H, int G,
                                                       int r, int dv) {
  __shared__ float x[1024];
  const int b = blockIdx.x, h = blockIdx.y;
  const int g = (h * G) / H;
  for (int i = threadIdx.x; i < r; i += blockDim.x) x[i] = o_lat[((size_t)b * H + h) * r + i];
  __syncthreads();
  const T* W = w_uv + (size_t)g * r * dv;
  for (int n = threadIdx.x; n < dv; n += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < r; ++k) acc += x[k] * Elem<T>::load(W, (size_t)k * dv + n);
    out[((size_t)b * H + h) * dv + n] = acc;
  }
}

hipError_t launch_out_proj(const Cfg& c, int batch, const float* o_lat, const void* w_uv,
                           float* out, hipStream_t s) {
  if (c.dtype == QKMLA_BF16)
    out_proj_kernel<uint16_t><<<dim3(batch, c.H), 256, 0, s>>>(o_lat, (const uint16_t*)w_uv, out,
                                                               c.H, c.G, c.r, c.dv);
  else
    out_proj_kernel<float><<<dim3(batch, c.H), 256, 0, s>>>(o_lat, (const float*)w_uv, out, c.H,
                                                            c.G, c.r, c.dv);
  return hipGetLastError();
}

}  // namespace qkmla
