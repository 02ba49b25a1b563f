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

// The log-sum-exp merge.  WPH wavefronts share head h of virtual sequence
// b; a block holds max(4, WPH) wavefronts, so 4 / WPH heads when WPH < 4, and
// covers r / ZD of the latent dims (grid z: which part).  The block first
// lists the sequence's partial slots in LDS (the slot each workgroup holding
// its tiles wrote, one thread per workgroup, so the slot arithmetic is off the
// load path).  Wave w of a head folds the sources w, w + WPH, ... with a
// running maximum, kMergeBatch at a time with all of their loads in flight;
// lane l holds 8 / ZD latent dims, one 16 / ZD-byte piece of the source's
// bf16 O row (r = 512).  The WPH waves of a head meet in LDS.  The host picks
// WPH (at most 8) so that a wave folds about kMergeBatch sources, and ZD = 2 when the
// sequences and heads alone give fewer blocks than CUs: the kernel's time is
// then about one round of loads, spread over the whole chip.  The tile prefix
// of the plan comes from the workspace, where the split-KV kernel left it.
constexpr int kMergeBatch = 8;     // sources in flight per wave (8 measured faster than 4 or 16)
constexpr int kMergeList = 1024;   // sources listed per pass

template <int WPH, int ZD>
__global__ __launch_bounds__((WPH < 4 ? 4 : WPH) * 64) void merge_kernel(
    const int32_t* __restrict__ plan, int B, int H, int r, int n_wg,
    const char* __restrict__ part, float* __restrict__ o_lat, float* __restrict__ lse) {
  static_assert(ZD == 1 || ZD == 2, "one or two parts of the latent dims");
  constexpr int kWaves = WPH < 4 ? 4 : WPH;
  constexpr int kHeads = kWaves / WPH;  // heads per block
  constexpr int kDl = 8 / ZD;           // latent dims per lane
  __shared__ int src[kMergeList];       // slot index p * kSlotsPerWg + slot, or -1 (nothing written)
  __shared__ f32x4 red[WPH > 1 ? kWaves : 1][kDl / 4][64];
  __shared__ float red_m[kWaves], red_l[kWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = blockIdx.y * kHeads + wave / WPH;  // this wave's head
  const int wi = wave % WPH;                        // its index among the head's waves
  const int d0 = blockIdx.z * (r / ZD) + kDl * lane;  // the lane's first latent dim
  float* out = o_lat + ((size_t)b * H + h) * r + d0;
  const bool lse_block = blockIdx.z == 0;
  const int Pb = plan[b], Pb1 = plan[b + 1];
  if (Pb1 == Pb) {  // invalid length: zeros and lse = -inf
    if (wi == 0) {
#pragma unroll
      for (int q = 0; q < kDl / 4; ++q) *(f32x4*)(out + 4 * q) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0 && lse && lse_block) lse[(size_t)b * H + h] = -INFINITY;
    }
    return;
  }
  const int64_t N = plan[B];
  const int p_lo = wg_of(Pb, N, n_wg);
  const int p_hi = wg_of(Pb1 - 1, N, n_wg);
  if (p_lo == p_hi) return;  // written directly by the decode kernel
  const size_t slot_bytes = kPartialSlotBytes(H, r);
  const size_t o_off = (size_t)H * 8 + ((size_t)h * r + d0) * 2;
  float M = -INFINITY, lsum = 0.f;
  f32x4 acc[kDl / 4];
#pragma unroll
  for (int q = 0; q < kDl / 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_src = p_hi - p_lo + 1;
  const int first = p_lo * kSlotsPerWg + merge_slot_of(Pb, p_lo, N, n_wg, p_lo);
  for (int c0 = 0; c0 < n_src; c0 += kMergeList) {
    const int cn = min(kMergeList, n_src - c0);
    // Workgroups between p_lo and p_hi with an empty range (more workgroups
    // than tiles) wrote nothing and are skipped.
    for (int i = tid; i < cn; i += kWaves * 64) {
      const int p = p_lo + c0 + i;
      const int slot = merge_slot_of(Pb, p_lo, N, n_wg, p);
      src[i] = slot < 0 ? -1 : p * kSlotsPerWg + slot;
    }
    __syncthreads();
    for (int k0 = wi; k0 < cn; k0 += kMergeBatch * WPH) {
      // Branch-free: an entry past the list or without a partial reads the
      // first workgroup's slot (always written) and gets weight 0, so the
      // loads of all kMergeBatch sources are issued before the first fold.
      float m[kMergeBatch], l[kMergeBatch];
      uint32_t ob[kMergeBatch][kDl / 2];
      bool ok[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int k = k0 + u * WPH;
        const int e = src[k < cn ? k : cn - 1];
        ok[u] = k < cn && e >= 0;
        const char* sp = part + (size_t)(ok[u] ? e : first) * slot_bytes;
        m[u] = ((const float*)sp)[h];
        l[u] = ((const float*)sp)[H + h];
        if constexpr (ZD == 1) {
          const uint4 v = *(const uint4*)(sp + o_off);
          ob[u][0] = v.x; ob[u][1] = v.y; ob[u][2] = v.z; ob[u][3] = v.w;
        } else {
          const uint2 v = *(const uint2*)(sp + o_off);
          ob[u][0] = v.x; ob[u][1] = v.y;
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the folds
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float Mn = ok[u] ? fmaxf(M, m[u]) : M;
        const float keep = Mn == M ? 1.f : exp2f(M - Mn);  // also M = Mn = -inf
        const float w = ok[u] ? exp2f(m[u] - Mn) : 0.f;
#pragma unroll
        for (int q = 0; q < kDl / 4; ++q) {
          const f32x4 v = {__uint_as_float(ob[u][2 * q] << 16),
                           __uint_as_float(ob[u][2 * q] & 0xFFFF0000u),
                           __uint_as_float(ob[u][2 * q + 1] << 16),
                           __uint_as_float(ob[u][2 * q + 1] & 0xFFFF0000u)};
          acc[q] = acc[q] * keep + v * w;
        }
        lsum = lsum * keep + l[u] * w;
        M = Mn;
      }
    }
    if (c0 + kMergeList < n_src) __syncthreads();  // the list is rewritten by the next pass
  }
  if constexpr (WPH > 1) {
#pragma unroll
    for (int q = 0; q < kDl / 4; ++q) red[wave][q][lane] = acc[q];
    if (lane == 0) {
      red_m[wave] = M;
      red_l[wave] = lsum;
    }
    __syncthreads();
    if (wi != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < WPH; ++k) Mt = fmaxf(Mt, red_m[wave + k]);
    f32x4 t[kDl / 4];
#pragma unroll
    for (int q = 0; q < kDl / 4; ++q) t[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int k = 0; k < WPH; ++k) {
      const float mk = red_m[wave + k];
      if (mk == -INFINITY) continue;  // a wave that held no source
      const float w = exp2f(mk - Mt);
#pragma unroll
      for (int q = 0; q < kDl / 4; ++q) t[q] += red[wave + k][q][lane] * w;
      lt += red_l[wave + k] * w;
    }
#pragma unroll
    for (int q = 0; q < kDl / 4; ++q) acc[q] = t[q];
    lsum = lt;
    M = Mt;
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int q = 0; q < kDl / 4; ++q) *(f32x4*)(out + 4 * q) = acc[q] * inv;
  if (lane == 0 && lse && lse_block) lse[(size_t)b * H + h] = (M + log2f(lsum)) * kLn2;
}

template <int WPH, int ZD>
static hipError_t launch_merge_wph(int nv, int H, int r, int n_wg, const int32_t* plan,
                             const char* part, float* o_lat, float* lse, hipStream_t s) {
  constexpr int kWaves = WPH < 4 ? 4 : WPH;
  constexpr int kHeads = kWaves / WPH;
  return launch_kernel(merge_kernel<WPH, ZD>, dim3(nv, H / kHeads, ZD), dim3(kWaves * 64), s,
                       plan, nv, H, r, n_wg, part, o_lat, lse);
}

template <int ZD>
static hipError_t launch_merge_zd(int wph, int nv, int H, int r, int n_wg, const int32_t* plan,
                                  const char* part, float* o_lat, float* lse, hipStream_t s) {
  switch (wph) {
    case 1: return launch_merge_wph<1, ZD>(nv, H, r, n_wg, plan, part, o_lat, lse, s);
    case 2: return launch_merge_wph<2, ZD>(nv, H, r, n_wg, plan, part, o_lat, lse, s);
    case 4: return launch_merge_wph<4, ZD>(nv, H, r, n_wg, plan, part, o_lat, lse, s);
    default: return launch_merge_wph<8, ZD>(nv, H, r, n_wg, plan, part, o_lat, lse, s);
  }
}

hipError_t launch_merge(const Cfg& c, int batch, int s_q, const WsLayout& ws, void* workspace,
                        int n_wg, float* o_lat, float* lse, hipStream_t s) {
  char* wsb = (char*)workspace;
  const int nv = batch * s_q;  // virtual sequences
  if (c.r != 8 * 64 || c.H % 4 != 0) return hipErrorInvalidValue;  // one 16-byte piece per lane
  // Sources of a sequence: the workgroups its tiles span, about n_wg / nv + 1
  // when the lengths are even.  WPH = the power of two that gives each wave
  // about kMergeBatch of them, at most 8 waves per head (a wave then folds
  // several batches: at one sequence of 256 workgroups, 4 x 8 sources).
  // (a sequence of exactly n_wg / nv workgroups' tiles has no extra source)
  const int per_seq = n_wg % nv == 0 ? n_wg / nv : n_wg / nv + 2;
  int wph = 1;
  while (wph < 8 && wph * kMergeBatch < per_seq) wph *= 2;
  const int32_t* plan = (const int32_t*)(wsb + ws.plan);
  const char* part = (const char*)(wsb + ws.partials);
  const int heads_per_block = wph < 4 ? 4 / wph : 1;
  const long blocks = (long)nv * (c.H / heads_per_block);
  if (blocks < 256)  // too few to fill the CUs: split the latent dims in two
    return launch_merge_zd<2>(wph, nv, c.H, c.r, n_wg, plan, part, o_lat, lse, s);
  return launch_merge_zd<1>(wph, nv, c.H, c.r, n_wg, plan, part, o_lat, lse, s);
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

// bf16 weights, 16 heads per KV group: one block per (b, g, 32 outputs),
// o[16 heads][32] = o_lat[16][r] . W^UV_g[r][32 columns] on
// mfma_f32_16x16x32_bf16 (o_lat rounded to bf16 for the A operand, fp32
// accumulation).  Wave w takes the K range [w r/4, (w+1) r/4): it stages its
// own 128 x 32 slice of W^UV_g in LDS (every load in flight at once), reads it
// back with ds_read_b64_tr_b16, which turns the row-major [k][n] layout into
// the k-contiguous B operand (in each 16-lane group lane i receives element
// i%4 of the 8-byte loads of lanes 4e + i/4, so lane 4e + q reads row k0+e,
// columns 4q..4q+3, and lane i ends with rows k0..k0+3 of column i), and the
// four partial sums meet in LDS in a fixed order.  Many small blocks: the
// projection of one sequence is a few hundred KB of weights, and spreading it
// over 4 G workgroups keeps each one's load to one round trip.
// Layouts (gfx950, 16x16x32): A lane l holds A[m=l%16][k=8(l/16)+j], B lane l
// holds B[k=8(l/16)+j][n=l%16], D lane l reg i holds D[4(l/16)+i][l%16].
constexpr int kOpK = 128;    // K rows per wave (r = 4 kOpK = 512)
constexpr int kOpN = 32;     // output columns per block

__global__ __launch_bounds__(256) void out_proj_mfma_kernel(const float* __restrict__ o_lat,
                                                            const uint16_t* __restrict__ w_uv,
                                                            float* __restrict__ out, int H,
                                                            int r, int dv) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[4][kOpK][kOpN];  // 32 KB
  __shared__ f32x4 red[3][2][64];
  const int b = blockIdx.x, g = blockIdx.y, n0 = blockIdx.z * kOpN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h0 = g * 16;
  const int m = lane & 15, kq = lane >> 4;
  const int kw = wave * kOpK;  // this wave's first K row
  const uint16_t* W = w_uv + (size_t)g * r * dv;
  const float* A = o_lat + ((size_t)b * H + h0 + m) * r + kw;
  // the wave's slice: 128 rows x 4 chunks of 16 B = 512 chunks, 8 per lane
  uint4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = lane + 64 * u, row = c >> 2, c8 = (c & 3) * 8;
    v[u] = n0 + c8 < dv ? *(const uint4*)(W + (size_t)(kw + row) * dv + n0 + c8)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
  f32x4 a[kOpK / 32][2];
#pragma unroll
  for (int ks = 0; ks < kOpK / 32; ++ks) {
    a[ks][0] = *(const f32x4*)(A + ks * 32 + kq * 8);
    a[ks][1] = *(const f32x4*)(A + ks * 32 + kq * 8 + 4);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = lane + 64 * u, row = c >> 2, c8 = (c & 3) * 8;
    *(uint4*)&wt[wave][row][c8] = v[u];
  }
  __syncthreads();
  const int e = (lane & 15) >> 2, q = lane & 3;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < kOpK / 32; ++ks) {
    const f32x4 a0 = a[ks][0], a1 = a[ks][1];
    const bf16x8 av = {(__bf16)a0[0], (__bf16)a0[1], (__bf16)a0[2], (__bf16)a0[3],
                       (__bf16)a1[0], (__bf16)a1[1], (__bf16)a1[2], (__bf16)a1[3]};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = nb * 16 + 4 * q;
      const int row = ks * 32 + kq * 8 + e;
      const bf16x4 lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &wt[wave][row][col]));
      const bf16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, &wt[wave][row + 4][col]));
      const bf16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
    }
  }
  if (wave > 0) {
    red[wave - 1][0][lane] = acc[0];
    red[wave - 1][1][lane] = acc[1];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const f32x4 t = ((acc[nb] + red[0][nb][lane]) + red[1][nb][lane]) + red[2][nb][lane];
    const int n = n0 + nb * 16 + m;
    if (n < dv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[((size_t)b * H + h0 + 4 * kq + i) * dv + n] = t[i];
    }
  }
}

bool out_proj_uses_mfma(const Cfg& c) {
  return c.dtype == QKMLA_BF16 && c.hpg == 16 && c.r == 4 * kOpK && c.dv % 16 == 0;
}

hipError_t launch_out_proj(const Cfg& c, int batch, const float* o_lat, const void* w_uv,
                           float* out, hipStream_t s) {
  if (out_proj_uses_mfma(c)) {
    out_proj_mfma_kernel<<<dim3(batch, c.G, (c.dv + kOpN - 1) / kOpN), 256, 0, s>>>(
        o_lat, (const uint16_t*)w_uv, out, c.H, c.r, c.dv);
  } else if (c.dtype == QKMLA_BF16)
    out_proj_kernel<uint16_t><<<dim3(batch, c.H), 256, 0, s>>>(o_lat, (const uint16_t*)w_uv, out,
                                                               c.H, c.G, c.r, c.dv);
  else
    out_proj_kernel<float><<<dim3(batch, c.H), 256, 0, s>>>(o_lat, (const float*)w_uv, out, c.H,
                                                            c.G, c.r, c.dv);
  return hipGetLastError();
}

}  // namespace qkmla
