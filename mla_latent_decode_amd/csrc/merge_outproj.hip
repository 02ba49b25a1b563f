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

// One block per (sequence b, head h, block of 128 latent dims); 256 threads =
// 8 source groups x 32 dim-quads.  Source group k combines the partials
// p = p_lo + k, p_lo + k + 8, ...; the eight partial sums meet in LDS.
constexpr int kMergeDims = 128;
constexpr int kMergeGroups = 8;

__global__ __launch_bounds__(256) void merge_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                    int L_cap, int H, int r, int n_wg,
                                                    const float* __restrict__ part,
                                                    float* __restrict__ o_lat,
                                                    float* __restrict__ lse) {
  __shared__ int P[kMaxBatch + 1];
  __shared__ f32x4 red[kMergeGroups][32];
  __shared__ float red_m[kMergeGroups], red_l[kMergeGroups];
  build_tile_prefix(seq_lens, B, L_cap, P);
  const int b = blockIdx.x, h = blockIdx.y, dblk = blockIdx.z;
  const int tid = threadIdx.x, sg = tid >> 5, dq = tid & 31;
  const int d0 = dblk * kMergeDims + 4 * dq;
  float* out = o_lat + ((size_t)b * H + h) * r + d0;
  const int n_b = P[b + 1] - P[b];
  if (n_b == 0) {  // invalid length: zeros and lse = -inf
    if (sg == 0) *(f32x4*)out = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid == 0 && dblk == 0 && lse) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const int64_t N = P[B];
  const int p_lo = wg_of(P[b], N, n_wg);
  const int p_hi = wg_of(P[b + 1] - 1, N, n_wg);
  if (p_lo == p_hi) return;  // written directly by the decode kernel
  const size_t slot_floats = (size_t)H * (r + 2);
  // Workgroups between p_lo and p_hi with an empty range (more workgroups
  // than tiles) wrote nothing and are skipped.
  auto slot = [&](int p) -> const float* {
    return part + ((size_t)p * kSlotsPerWg + merge_slot(P, b, N, n_wg, p)) * slot_floats;
  };
  auto empty = [&](int p) { return merge_slot(P, b, N, n_wg, p) < 0; };
  // pass 1: M = max_s m_s
  float M = -INFINITY;
  for (int p = p_lo + tid; p <= p_hi; p += 256)
    if (!empty(p)) M = fmaxf(M, slot(p)[h]);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((tid & 63) == 0) red_m[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  // pass 2: weighted sums
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int p = p_lo + sg; p <= p_hi; p += kMergeGroups) {
    if (empty(p)) continue;
    const float* sp = slot(p);
    const float w = exp2f(sp[h] - M);
    lsum += w * sp[H + h];
    const f32x4 v = *(const f32x4*)(sp + 2 * H + (size_t)h * r + d0);
    acc += w * v;
  }
  red[sg][dq] = acc;
  if (dq == 0) red_l[sg] = lsum;
  __syncthreads();
  if (sg == 0) {
    f32x4 t = red[0][dq];
    float l = red_l[0];
#pragma unroll
    for (int k = 1; k < kMergeGroups; ++k) {
      t += red[k][dq];
      l += red_l[k];
    }
    const float inv = 1.0f / l;
    *(f32x4*)out = t * inv;
    if (dq == 0 && dblk == 0 && lse) lse[(size_t)b * H + h] = (M + log2f(l)) * kLn2;
  }
}

hipError_t launch_merge(const Cfg& c, int batch, const int32_t* seq_lens, int L_cap,
                        const WsLayout& ws, void* workspace, int n_wg, float* o_lat, float* lse,
                        hipStream_t s) {
  char* wsb = (char*)workspace;
  merge_kernel<<<dim3(batch, c.H, c.r / kMergeDims), 256, 0, s>>>(
      seq_lens, batch, L_cap, c.H, c.r, n_wg, (const float*)(wsb + ws.partials), o_lat, lse);
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
