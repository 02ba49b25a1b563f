// Training / prefill of QK-Normed MLA in the explicit form: causal attention
// over whole sequences with materialised, RMS-normalised keys, forward and
// backward ("QK-Normed MLA: QK normalization without full key caching",
// technical summary, Methodology: RMSNorm decomposition and Blockwise
// Normalization; Results: the models are trained in this form).
//
// Row-parallel kernels for any layer shape and either storage type.  Every
// intermediate is fp32 in the workspace; every gradient is fp32.
//
// Forward, per sequence b, token i, head h in group g (positions are token
// indices):
//   K^_{j,g} = [RMSNorm_{gk}(c_j W^UK_g) | RoPE_j(RMSNorm_{gkr}(k^R_j))]
//   Q^_{i,h} = [RMSNorm_{gq}(q^C_{i,h})  | RoPE_i(RMSNorm_{gqr}(q^R_{i,h}))]
//   V_{j,g}  = c_j W^UV_g
//   s_{ij} = tau Q^_{i,h} . K^_{j,g} (j <= i),  o_{i,h} = sum_j softmax_j(s) V_{j,g}
// Backward (loss gradient d_o): D_i = d_o_i . o_i, p_ij = exp(s_ij - lse_i),
//   ds_ij = p_ij (d_o_i . V_j - D_i);  dQ^_i = tau sum_j ds_ij K^_j;
//   dK^_j = tau sum_{i,h in g} ds_ij Q^_i;  dV_j = sum_{i,h in g} p_ij d_o_i;
// then back through RoPE (the transposed rotation), the RMSNorms
// (y = gamma x a with a = 1/S(x):  dx = a gamma dy - x a^3 (sum gamma dy x)/n,
// dgamma = sum dy x a) and the up-projections.
#include "device_common.h"
#include "qkmla_internal.h"

namespace qkmla {

namespace {

constexpr int kChunk = 256;   // keys (queries) per chunk of the attention kernels
constexpr int kKvTok = 8;     // tokens per workgroup of the key/value projection
constexpr int kLatTok = 4;    // tokens per workgroup of the latent gradient
constexpr int kWgRows = 16;   // latent rows per workgroup of the weight gradients
constexpr int kWgTok = 32;    // tokens per LDS chunk of the weight gradients
constexpr int kGammaSplit = 512;  // most row ranges of the RMSNorm weight gradients
static_assert(kGammaSplit % 16 == 0, "gamma_final_kernel gives each of 16 lanes a share");

// Row ranges for an RMSNorm weight gradient over `rows` rows: about 128 rows
// each, a multiple of 16, at least 16 and at most kGammaSplit.
static int gamma_splits(int rows) {
  const int want = ((rows + 127) / 128 + 15) / 16 * 16;
  return want < 16 ? 16 : want > kGammaSplit ? kGammaSplit : want;
}

// Token rows are packed: sequence s holds rows [start_s, start_s + len_s).
struct TrainDims {
  int n_rows, n_seq, max_len, H, G, r, dc, dr, dv, dqk, hpg;
  int qk_norm;
  float eps, tau, base;
  const float2* rope_cs;  // [max_len][d_r/2]: (cos, sin) of the angle of position t, pair i
  const int32_t* rpos;    // [n_rows] position of the row in its sequence
  const int32_t* rlen;    // [n_rows] length of the row's sequence
};

TrainDims dims_of(const Cfg& c, const TrainSeqs& q, const float2* rope_cs, const int32_t* rpos,
                  const int32_t* rlen) {
  return TrainDims{q.n_rows, q.n_seq, q.max_len, c.H, c.G, c.r, c.dc, c.dr, c.dv, c.dc + c.dr,
                   c.hpg, c.qk_norm, c.eps, c.tau, c.base, rope_cs, rpos, rlen};
}

// ---- sequence tables --------------------------------------------------------
// seq_table_kernel: per sequence s, its start and length from the caller's
// cu_seqlens (or, with cu == nullptr, equal lengths max_len), clamped so that
// 0 <= start, start + len <= n_rows and len <= max_len; a clamp, a gap or an
// overlap sets QKMLA_DEV_BAD_SEQ_LEN (the outputs are then undefined, every
// access stays in bounds).
__global__ __launch_bounds__(256) void seq_table_kernel(int n_seq, const int32_t* __restrict__ cu,
                                                        int n_rows, int max_len,
                                                        int2* __restrict__ seqs,
                                                        int32_t* __restrict__ status) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n_seq) return;
  int a = cu ? cu[s] : s * max_len, b = cu ? cu[s + 1] : (s + 1) * max_len;
  bool bad = cu && ((s == 0 && a != 0) || (s == n_seq - 1 && b != n_rows));
  const int start = min(max(a, 0), n_rows);
  const int end = min(max(b, start), n_rows);
  const int len = min(end - start, max_len);
  bad |= start != a || end != b || len != end - start;
  seqs[s] = make_int2(start, len);
  if (bad && status) atomicOr(status, QKMLA_DEV_BAD_SEQ_LEN);
}

// Rows first become one-token sequences of their own; then every sequence
// claims its rows.  A row ends with rpos <= row and row - rpos + rlen <= n_rows
// whatever cu held.
__global__ __launch_bounds__(256) void row_init_kernel(int n_rows, int32_t* __restrict__ rpos,
                                                       int32_t* __restrict__ rlen) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n_rows) return;
  rpos[r] = 0;
  rlen[r] = 1;
}

__global__ __launch_bounds__(256) void row_fill_kernel(const int2* __restrict__ seqs,
                                                       int32_t* __restrict__ rpos,
                                                       int32_t* __restrict__ rlen) {
  const int2 sl = seqs[blockIdx.x];
  for (int t = threadIdx.x; t < sl.y; t += 256) {
    rpos[sl.x + t] = t;
    rlen[sl.x + t] = sl.y;
  }
}

// The RoPE angles of every position once per call (each is used by every
// head and group of that position, forward and backward).
__global__ __launch_bounds__(256) void rope_table_kernel(int T, int dr, float base, float2* cs) {
  const int half = dr / 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * half) return;
  float c, s;
  rope_cos_sin((int)(i / half), (int)(i % half), dr, base, &c, &s);
  cs[i] = make_float2(c, s);
}

__device__ __forceinline__ void rope_at(const TrainDims& d, int pos, int i, float* c, float* s) {
  const float2 t = d.rope_cs[(size_t)pos * (d.dr / 2) + i];
  *c = t.x;
  *s = t.y;
}

// Sum over the block (blockDim.x = 256); `red` holds 4 floats.  Every thread
// gets the total.
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---- forward: normalised, rotated queries ----------------------------------
// One wavefront per (token row, head).  Qh[row][h] = [q^ content | q^R], and
// the inverse RMS values for the backward.
// MF: write the bf16 operand of the MFMA attention instead (same layout,
// scaled by tau*log2(e)).
template <typename T, bool MF>
__global__ __launch_bounds__(256) void prep_q_kernel(TrainDims d, const T* __restrict__ q_c,
                                                     const T* __restrict__ q_rope,
                                                     const float* __restrict__ gq,
                                                     const float* __restrict__ gqr,
                                                     float* __restrict__ Qh,
                                                     uint16_t* __restrict__ Qb,
                                                     float* __restrict__ aq,
                                                     float* __restrict__ aqr) {
  const size_t row = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (h >= d.H) return;
  const int pos = d.rpos[row];
  const size_t qh = row * d.H + h;
  const T* qc = q_c + qh * d.dc;
  const T* qr = q_rope + qh * d.dr;
  const float qs = d.tau * kLog2e;
  auto put = [&](int e, float v) {
    if constexpr (MF) Qb[qh * d.dqk + e] = f32_to_bf16(v * qs);
    else Qh[qh * d.dqk + e] = v;
  };
  float a = 1.f, ar = 1.f;
  if (d.qk_norm) {
    float ss = 0.f, sr = 0.f;
    for (int e = lane; e < d.dc; e += 64) {
      const float v = Elem<T>::load(qc, e);
      ss += v * v;
    }
    for (int e = lane; e < d.dr; e += 64) {
      const float v = Elem<T>::load(qr, e);
      sr += v * v;
    }
    a = 1.0f / sqrtf(wave_sum(ss) / (float)d.dc + d.eps);
    ar = 1.0f / sqrtf(wave_sum(sr) / (float)d.dr + d.eps);
    if (lane == 0) {
      aq[qh] = a;
      aqr[qh] = ar;
    }
  }
  for (int e = lane; e < d.dc; e += 64)
    put(e, Elem<T>::load(qc, e) * (d.qk_norm ? gq[e] * a : 1.f));
  for (int i = lane; i < d.dr / 2; i += 64) {
    float x0 = Elem<T>::load(qr, 2 * i), x1 = Elem<T>::load(qr, 2 * i + 1);
    if (d.qk_norm) {
      x0 *= gqr[2 * i] * ar;
      x1 *= gqr[2 * i + 1] * ar;
    }
    float cs, sn;
    rope_at(d, pos, i, &cs, &sn);
    put(d.dc + 2 * i, x0 * cs - x1 * sn);
    put(d.dc + 2 * i + 1, x0 * sn + x1 * cs);
  }
}

// The same for the MFMA attention's shape (bf16, d_c = 128, d_r = 64), with
// 16-byte accesses.  A wave takes kMfHeads = 8 heads of one row: lane l holds
// content dims 8(l%16)..8(l%16)+7 of heads l/16 and 4 + l/16, and RoPE dims
// 8(l%8)..8(l%8)+7 (four pairs) of head l/8, so every load and store moves
// 16 bytes per lane and the RMS sums close within 16- and 8-lane groups.  The
// gammas and the rotation of the row's position are loaded once per wave.
// Needs q_c, q_rope and both gammas 16-byte aligned (checked by the launcher).
constexpr int kMfHeads = 8;  // heads per wave of the vector row kernels

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 f32_to_bf16x8(const float* y) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = f32_to_bf16(y[2 * i]) | ((uint32_t)f32_to_bf16(y[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Sum over aligned groups of `width` lanes (a power of two up to 16).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(256) void prep_q_mf_kernel(TrainDims d,
                                                        const uint16_t* __restrict__ q_c,
                                                        const uint16_t* __restrict__ q_rope,
                                                        const float* __restrict__ gq,
                                                        const float* __restrict__ gqr,
                                                        uint16_t* __restrict__ Qb,
                                                        float* __restrict__ aq,
                                                        float* __restrict__ aqr) {
  static_assert(kMfHeads == 8, "the lane map covers eight heads");
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int h0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * kMfHeads;
  if (h0 >= d.H) return;
  const int c16 = lane & 15, c8 = lane & 7;
  const size_t qa = row * d.H + h0 + (lane >> 4);  // content head of the first load
  const size_t qr = row * d.H + h0 + (lane >> 3);  // RoPE head
  const uint4 va = *(const uint4*)(q_c + qa * 128 + 8 * c16);
  const uint4 vb = *(const uint4*)(q_c + (qa + 4) * 128 + 8 * c16);
  const uint4 vr = *(const uint4*)(q_rope + qr * 64 + 8 * c8);
  float g[8], gr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = gr[i] = 1.f;
  if (d.qk_norm) {
    const f32x4 g0 = *(const f32x4*)(gq + 8 * c16), g1 = *(const f32x4*)(gq + 8 * c16 + 4);
    const f32x4 r0 = *(const f32x4*)(gqr + 8 * c8), r1 = *(const f32x4*)(gqr + 8 * c8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] = g0[i];
      g[4 + i] = g1[i];
      gr[i] = r0[i];
      gr[4 + i] = r1[i];
    }
  }
  // rotation of pairs 4 c8 .. 4 c8 + 3 at the row's position
  const float4* cs4 = (const float4*)(d.rope_cs + (size_t)d.rpos[row] * 32 + 4 * c8);
  const float4 t0 = cs4[0], t1 = cs4[1];
  const float cs[4] = {t0.x, t0.z, t1.x, t1.z}, sn[4] = {t0.y, t0.w, t1.y, t1.w};
  const float qs = d.tau * kLog2e;
  float x[8], y[8];
  // content, heads h0 + l/16 and h0 + 4 + l/16
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8_to_f32(half ? vb : va, x);
    float a = 1.f;
    if (d.qk_norm) {
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
      a = 1.0f / sqrtf(group_sum<16>(sq) / 128.f + d.eps);
      if (c16 == 0) aq[qa + 4 * half] = a;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (d.qk_norm ? x[e] * (g[e] * a) : x[e]) * qs;
    *(uint4*)(Qb + (qa + 4 * half) * 192 + 8 * c16) = f32_to_bf16x8(y);
  }
  // RoPE part, head h0 + l/8
  bf16x8_to_f32(vr, x);
  float ar = 1.f;
  if (d.qk_norm) {
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
    ar = 1.0f / sqrtf(group_sum<8>(sq) / 64.f + d.eps);
    if (c8 == 0) aqr[qr] = ar;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = x[2 * i], x1 = x[2 * i + 1];
    if (d.qk_norm) {
      x0 *= gr[2 * i] * ar;
      x1 *= gr[2 * i + 1] * ar;
    }
    y[2 * i] = (x0 * cs[i] - x1 * sn[i]) * qs;
    y[2 * i + 1] = (x0 * sn[i] + x1 * cs[i]) * qs;
  }
  *(uint4*)(Qb + qr * 192 + 128 + 8 * c8) = f32_to_bf16x8(y);
}

// ---- forward: keys and values -----------------------------------------------
// Workgroup = kKvTok token rows x one group g.  Thread e owns output dim e of
// k = c W^UK_g and v = c W^UV_g for the workgroup's tokens.  Writes the raw
// key (for the backward), the normalised key with the normalised, rotated
// RoPE key after it, the value, and the inverse RMS values.
template <typename T>
__global__ __launch_bounds__(256) void prep_kv_kernel(
    TrainDims d, int n_rows, const T* __restrict__ c, const T* __restrict__ k_rope,
    const float* __restrict__ w_uk, const T* __restrict__ w_uv, const float* __restrict__ gk,
    const float* __restrict__ gkr, float* __restrict__ Kh, float* __restrict__ Kraw,
    float* __restrict__ V, float* __restrict__ ak, float* __restrict__ akr) {
  extern __shared__ float lds[];  // c rows [kKvTok][r], then kKvTok * 8 reduction slots
  float* cs = lds;
  float* red = lds + kKvTok * d.r;
  const size_t row0 = (size_t)blockIdx.x * kKvTok;
  const int g = blockIdx.y, tid = threadIdx.x;
  const int ntok = (int)min((size_t)kKvTok, (size_t)n_rows - row0);
  auto put_k = [&](size_t row, int e, float v) { Kh[(row * d.G + g) * d.dqk + e] = v; };
  for (int i = tid; i < kKvTok * d.r; i += 256) {
    const int tk = i / d.r, e = i % d.r;
    cs[i] = tk < ntok ? Elem<T>::load(c, (row0 + tk) * d.r + e) : 0.f;
  }
  __syncthreads();
  // content key: dims e = tid, tid + 256, ...; sum of squares per token
  float ssq[kKvTok];
#pragma unroll
  for (int t = 0; t < kKvTok; ++t) ssq[t] = 0.f;
  const float* wk = w_uk + (size_t)g * d.r * d.dc;
  for (int e = tid; e < d.dc; e += 256) {
    float acc[kKvTok];
#pragma unroll
    for (int t = 0; t < kKvTok; ++t) acc[t] = 0.f;
    for (int i = 0; i < d.r; ++i) {
      const float w = wk[(size_t)i * d.dc + e];
#pragma unroll
      for (int t = 0; t < kKvTok; ++t) acc[t] += cs[t * d.r + i] * w;
    }
#pragma unroll
    for (int t = 0; t < kKvTok; ++t) {
      ssq[t] += acc[t] * acc[t];
      if (t < ntok) Kraw[((row0 + t) * d.G + g) * d.dc + e] = acc[t];
    }
  }
  // per-token totals over the block (one reduction slot per wave and token)
#pragma unroll
  for (int t = 0; t < kKvTok; ++t) {
    const float s = wave_sum(ssq[t]);
    if ((tid & 63) == 0) red[t * 4 + (tid >> 6)] = s;
  }
  // value
  const T* wv = w_uv + (size_t)g * d.r * d.dv;
  for (int e = tid; e < d.dv; e += 256) {
    float acc[kKvTok];
#pragma unroll
    for (int t = 0; t < kKvTok; ++t) acc[t] = 0.f;
    for (int i = 0; i < d.r; ++i) {
      const float w = Elem<T>::load(wv, (size_t)i * d.dv + e);
#pragma unroll
      for (int t = 0; t < kKvTok; ++t) acc[t] += cs[t * d.r + i] * w;
    }
#pragma unroll
    for (int t = 0; t < kKvTok; ++t)
      if (t < ntok) V[((row0 + t) * d.G + g) * d.dv + e] = acc[t];
  }
  __syncthreads();
  // normalised content key (reads back this thread's own raw values)
  for (int t = 0; t < ntok; ++t) {
    const size_t kg = (row0 + t) * d.G + g;
    const float a = d.qk_norm
                        ? 1.0f / sqrtf((red[t * 4] + red[t * 4 + 1] + red[t * 4 + 2] +
                                        red[t * 4 + 3]) / (float)d.dc + d.eps)
                        : 1.f;
    if (tid == 0 && d.qk_norm) ak[kg] = a;
    for (int e = tid; e < d.dc; e += 256)
      put_k(row0 + t, e, Kraw[kg * d.dc + e] * (d.qk_norm ? gk[e] * a : 1.f));
  }
  // RoPE key: wave w handles tokens w, w + 4, ...
  const int wave = tid >> 6, lane = tid & 63;
  for (int t = wave; t < ntok; t += 4) {
    const size_t row = row0 + t;
    const int pos = d.rpos[row];
    const T* kr = k_rope + row * d.dr;
    float ar = 1.f;
    if (d.qk_norm) {
      float s = 0.f;
      for (int e = lane; e < d.dr; e += 64) {
        const float v = Elem<T>::load(kr, e);
        s += v * v;
      }
      ar = 1.0f / sqrtf(wave_sum(s) / (float)d.dr + d.eps);
      if (g == 0 && lane == 0) akr[row] = ar;
    }
    for (int i = lane; i < d.dr / 2; i += 64) {
      float x0 = Elem<T>::load(kr, 2 * i), x1 = Elem<T>::load(kr, 2 * i + 1);
      if (d.qk_norm) {
        x0 *= gkr[2 * i] * ar;
        x1 *= gkr[2 * i + 1] * ar;
      }
      float c0, s0;
      rope_at(d, pos, i, &c0, &s0);
      put_k(row, d.dc + 2 * i, x0 * c0 - x1 * s0);
      put_k(row, d.dc + 2 * i + 1, x0 * s0 + x1 * c0);
    }
  }
}

// ---- forward attention ---------------------------------------------------------
// One workgroup per (query row, head): exact online softmax over chunks of
// kChunk keys j <= i (exp2 domain).
__global__ __launch_bounds__(256) void attn_fwd_kernel(TrainDims d, const float* __restrict__ Qh,
                                                       const float* __restrict__ Kh,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ o,
                                                       float* __restrict__ lse) {
  extern __shared__ float lds[];  // q [dqk], p [kChunk], red [4]
  float* q = lds;
  float* p = lds + d.dqk;
  float* red = p + kChunk;
  const size_t row = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x, g = h / d.hpg;
  const int i = d.rpos[row];
  const size_t seq0 = row - i;  // first row of the sequence
  const float sc = d.tau * kLog2e;
  for (int e = tid; e < d.dqk; e += 256) q[e] = Qh[(row * d.H + h) * d.dqk + e] * sc;
  __syncthreads();
  float acc = 0.f, m_run = -INFINITY, l_run = 0.f;
  const int e_out = tid;  // output dim owned by this thread (d_v <= 256)
  for (int j0 = 0; j0 <= i; j0 += kChunk) {
    const int j = j0 + tid;
    float s = -INFINITY;
    if (j <= i) {
      const float* k = Kh + ((seq0 + j) * d.G + g) * d.dqk;
      float a = 0.f;
      for (int e = 0; e < d.dqk; ++e) a += q[e] * k[e];
      s = a;
    }
    const float m_new = fmaxf(m_run, block_max(s, red));
    const float f = exp2f(m_run - m_new);
    const float pv = j <= i ? exp2f(s - m_new) : 0.f;
    p[tid] = pv;
    l_run = l_run * f + block_sum(pv, red);
    m_run = m_new;
    const int n = min(kChunk, i + 1 - j0);
    if (e_out < d.dv) {
      float a = acc * f;
      for (int jj = 0; jj < n; ++jj) a += p[jj] * V[((seq0 + j0 + jj) * d.G + g) * d.dv + e_out];
      acc = a;
    }
    __syncthreads();
  }
  if (e_out < d.dv) o[(row * d.H + h) * d.dv + e_out] = acc / l_run;
  if (tid == 0) lse[row * d.H + h] = (m_run + log2f(l_run)) * kLn2;
}

// ---- backward attention: query side ---------------------------------------------
// One workgroup per (query row i, head h): D = d_o . o, then
// dQ^ = tau sum_j ds_ij K^_j over j <= i.
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(
    TrainDims d, const float* __restrict__ Qh, const float* __restrict__ Kh,
    const float* __restrict__ V, const float* __restrict__ o, const float* __restrict__ lse,
    const float* __restrict__ d_o, float* __restrict__ dQh, float* __restrict__ Dsum) {
  extern __shared__ float lds[];  // q [dqk], do [dv], ds [kChunk], red [4]
  float* q = lds;
  float* dov = q + d.dqk;
  float* ds = dov + d.dv;
  float* red = ds + kChunk;
  const size_t row = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x, g = h / d.hpg;
  const int i = d.rpos[row];
  const size_t seq0 = row - i;
  const size_t qh = row * d.H + h;
  for (int e = tid; e < d.dqk; e += 256) q[e] = Qh[qh * d.dqk + e];
  float dd = 0.f;
  for (int e = tid; e < d.dv; e += 256) {
    const float g_o = d_o[qh * d.dv + e];
    dov[e] = g_o;
    dd += g_o * o[qh * d.dv + e];
  }
  const float D = block_sum(dd, red);  // also orders the LDS writes above
  if (tid == 0) Dsum[qh] = D;
  const float L = lse[qh];
  float acc0 = 0.f, acc1 = 0.f;  // dims tid, tid + 256 (dqk <= 512)
  for (int j0 = 0; j0 <= i; j0 += kChunk) {
    const int j = j0 + tid;
    float v_ds = 0.f;
    if (j <= i) {
      const size_t kg = (seq0 + j) * d.G + g;
      const float* k = Kh + kg * d.dqk;
      float s = 0.f;
      for (int e = 0; e < d.dqk; ++e) s += q[e] * k[e];
      const float pj = expf(d.tau * s - L);
      const float* v = V + kg * d.dv;
      float dp = 0.f;
      for (int e = 0; e < d.dv; ++e) dp += dov[e] * v[e];
      v_ds = pj * (dp - D);
    }
    ds[tid] = v_ds;
    __syncthreads();
    const int n = min(kChunk, i + 1 - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float* k = Kh + ((seq0 + j0 + jj) * d.G + g) * d.dqk;
      const float w = ds[jj];
      if (tid < d.dqk) acc0 += w * k[tid];
      if (tid + 256 < d.dqk) acc1 += w * k[tid + 256];
    }
    __syncthreads();
  }
  if (tid < d.dqk) dQh[qh * d.dqk + tid] = d.tau * acc0;
  if (tid + 256 < d.dqk) dQh[qh * d.dqk + tid + 256] = d.tau * acc1;
}

// ---- backward attention: key/value side ------------------------------------------
// One workgroup per (key row j, group g): over the group's heads and queries
// i >= j, dK^_j = tau sum ds_ij Q^_i and dV_j = sum p_ij d_o_i.
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(
    TrainDims d, const float* __restrict__ Qh, const float* __restrict__ Kh,
    const float* __restrict__ V, const float* __restrict__ lse, const float* __restrict__ d_o,
    const float* __restrict__ Dsum, float* __restrict__ dKh, float* __restrict__ dV) {
  extern __shared__ float lds[];  // k [dqk], v [dv], p [kChunk], ds [kChunk]
  float* k = lds;
  float* v = k + d.dqk;
  float* p = v + d.dv;
  float* ds = p + kChunk;
  const size_t row = blockIdx.x;
  const int g = blockIdx.y, tid = threadIdx.x;
  const int j = d.rpos[row];
  const int L = d.rlen[row];
  const size_t seq0 = row - j;
  const size_t kg = row * d.G + g;
  for (int e = tid; e < d.dqk; e += 256) k[e] = Kh[kg * d.dqk + e];
  for (int e = tid; e < d.dv; e += 256) v[e] = V[kg * d.dv + e];
  __syncthreads();
  float dk0 = 0.f, dk1 = 0.f, dvv = 0.f;
  for (int hh = 0; hh < d.hpg; ++hh) {
    const int h = g * d.hpg + hh;
    for (int i0 = j; i0 < L; i0 += kChunk) {
      const int i = i0 + tid;
      float pv = 0.f, dsv = 0.f;
      if (i < L) {
        const size_t qh = (seq0 + i) * d.H + h;
        const float* q = Qh + qh * d.dqk;
        float s = 0.f;
        for (int e = 0; e < d.dqk; ++e) s += q[e] * k[e];
        pv = expf(d.tau * s - lse[qh]);
        const float* go = d_o + qh * d.dv;
        float dp = 0.f;
        for (int e = 0; e < d.dv; ++e) dp += go[e] * v[e];
        dsv = pv * (dp - Dsum[qh]);
      }
      p[tid] = pv;
      ds[tid] = dsv;
      __syncthreads();
      const int n = min(kChunk, L - i0);
      for (int ii = 0; ii < n; ++ii) {
        const size_t qh = (seq0 + i0 + ii) * d.H + h;
        const float* q = Qh + qh * d.dqk;
        const float w = ds[ii];
        if (tid < d.dqk) dk0 += w * q[tid];
        if (tid + 256 < d.dqk) dk1 += w * q[tid + 256];
        if (tid < d.dv) dvv += p[ii] * d_o[qh * d.dv + tid];
      }
      __syncthreads();
    }
  }
  if (tid < d.dqk) dKh[kg * d.dqk + tid] = d.tau * dk0;
  if (tid + 256 < d.dqk) dKh[kg * d.dqk + tid + 256] = d.tau * dk1;
  if (tid < d.dv) dV[kg * d.dv + tid] = dvv;
}

// RMSNorm backward of one row held by a wavefront: y = gamma x a (a = 1/S):
//   dx = a gamma dy - x a^3 (sum_j gamma_j dy_j x_j) / n.
// dy, x are read through the accessors; dx is written by `put`.
template <typename DY, typename X, typename PUT>
__device__ void rmsnorm_bwd_wave(int n, float a, const float* gamma, DY dy, X x, PUT put,
                                 int lane) {
  float s = 0.f;
  for (int e = lane; e < n; e += 64) s += gamma[e] * dy(e) * x(e);
  s = wave_sum(s);
  const float k = a * a * a * s / (float)n;
  for (int e = lane; e < n; e += 64) put(e, a * gamma[e] * dy(e) - x(e) * k);
}

// ---- backward: query norms and rotation -------------------------------------------
// One wavefront per (token row, head).  Each lane turns back (transposed
// rotation) the RoPE-part gradient of its own pairs, keeps it in registers
// for the RMSNorm backward and stores it over dQ^ for the gamma reduction.
template <typename T>
__global__ __launch_bounds__(256) void q_norm_bwd_kernel(
    TrainDims d, const T* __restrict__ q_c, const T* __restrict__ q_rope,
    const float* __restrict__ gq, const float* __restrict__ gqr, const float* __restrict__ aq,
    const float* __restrict__ aqr, float* __restrict__ dQh, float* __restrict__ d_q_c,
    float* __restrict__ d_q_rope) {
  const size_t row = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (h >= d.H) return;
  const int pos = d.rpos[row];
  const size_t qh = row * d.H + h;
  float* dy = dQh + qh * d.dqk;
  float* dyr = dy + d.dc;
  const T* xc = q_c + qh * d.dc;
  const T* xr = q_rope + qh * d.dr;
  float* oc = d_q_c + qh * d.dc;
  float* orr = d_q_rope + qh * d.dr;
  // content part
  if (d.qk_norm)
    rmsnorm_bwd_wave(
        d.dc, aq[qh], gq, [&](int e) { return dy[e]; },
        [&](int e) { return Elem<T>::load(xc, e); }, [&](int e, float v) { oc[e] = v; }, lane);
  else
    for (int e = lane; e < d.dc; e += 64) oc[e] = dy[e];
  // RoPE part: pairs lane, lane + 64 (d_r <= 256)
  float u0[2], u1[2];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    u0[k] = u1[k] = 0.f;
    if (i < d.dr / 2) {
      float cs, sn;
      rope_at(d, pos, i, &cs, &sn);
      const float y0 = dyr[2 * i], y1 = dyr[2 * i + 1];
      u0[k] = y0 * cs + y1 * sn;
      u1[k] = -y0 * sn + y1 * cs;
      dyr[2 * i] = u0[k];
      dyr[2 * i + 1] = u1[k];
      if (d.qk_norm)
        s += gqr[2 * i] * u0[k] * Elem<T>::load(xr, 2 * i) +
             gqr[2 * i + 1] * u1[k] * Elem<T>::load(xr, 2 * i + 1);
    }
  }
  if (!d.qk_norm) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = lane + 64 * k;
      if (i < d.dr / 2) {
        orr[2 * i] = u0[k];
        orr[2 * i + 1] = u1[k];
      }
    }
    return;
  }
  const float a = aqr[qh];
  const float kk = a * a * a * wave_sum(s) / (float)d.dr;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < d.dr / 2) {
      orr[2 * i] = a * gqr[2 * i] * u0[k] - Elem<T>::load(xr, 2 * i) * kk;
      orr[2 * i + 1] = a * gqr[2 * i + 1] * u1[k] - Elem<T>::load(xr, 2 * i + 1) * kk;
    }
  }
}

// The same for the MFMA attention's shape (bf16, d_c = 128, d_r = 64), with
// 16-byte accesses and the lane map of prep_q_mf_kernel: lane l holds content
// dims 8(l%16)..+7 of heads l/16 and 4 + l/16 and RoPE dims 8(l%8)..+7 of
// head l/8 of the wave's kMfHeads heads.  Needs q_c, q_rope, both gammas,
// d_q_c and d_q_rope 16-byte aligned (checked by the launcher).
__global__ __launch_bounds__(256) void q_norm_bwd_mf_kernel(
    TrainDims d, const uint16_t* __restrict__ q_c, const uint16_t* __restrict__ q_rope,
    const float* __restrict__ gq, const float* __restrict__ gqr, const float* __restrict__ aq,
    const float* __restrict__ aqr, float* __restrict__ dQh, float* __restrict__ d_q_c,
    float* __restrict__ d_q_rope) {
  static_assert(kMfHeads == 8, "the lane map covers eight heads");
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int h0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * kMfHeads;
  if (h0 >= d.H) return;
  const int c16 = lane & 15, c8 = lane & 7;
  const size_t qa = row * d.H + h0 + (lane >> 4);  // content heads qa, qa + 4
  const size_t qr = row * d.H + h0 + (lane >> 3);  // RoPE head
  f32x4 dy[2][2], dr[2];
  uint4 xc[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const float* p = dQh + (qa + 4 * half) * 192 + 8 * c16;
    dy[half][0] = *(const f32x4*)p;
    dy[half][1] = *(const f32x4*)(p + 4);
    xc[half] = *(const uint4*)(q_c + (qa + 4 * half) * 128 + 8 * c16);
  }
  float* pr = dQh + qr * 192 + 128 + 8 * c8;
  dr[0] = *(const f32x4*)pr;
  dr[1] = *(const f32x4*)(pr + 4);
  const uint4 xr = *(const uint4*)(q_rope + qr * 64 + 8 * c8);
  const float a_c[2] = {aq[qa], aq[qa + 4]}, a_r = aqr[qr];
  float g[8], gr[8];
  {
    const f32x4 g0 = *(const f32x4*)(gq + 8 * c16), g1 = *(const f32x4*)(gq + 8 * c16 + 4);
    const f32x4 r0 = *(const f32x4*)(gqr + 8 * c8), r1 = *(const f32x4*)(gqr + 8 * c8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] = g0[i];
      g[4 + i] = g1[i];
      gr[i] = r0[i];
      gr[4 + i] = r1[i];
    }
  }
  const float4* cs4 = (const float4*)(d.rope_cs + (size_t)d.rpos[row] * 32 + 4 * c8);
  const float4 t0 = cs4[0], t1 = cs4[1];
  const float cs[4] = {t0.x, t0.z, t1.x, t1.z}, sn[4] = {t0.y, t0.w, t1.y, t1.w};
  float x[8], y[8], o[8];
  // content: the RMSNorm backward of heads qa and qa + 4
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = dy[half][0][i];
      y[4 + i] = dy[half][1][i];
    }
    float* out = d_q_c + (qa + 4 * half) * 128 + 8 * c16;
    if (!d.qk_norm) {
      *(f32x4*)out = dy[half][0];
      *(f32x4*)(out + 4) = dy[half][1];
      continue;
    }
    bf16x8_to_f32(xc[half], x);
    float sp = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sp += g[e] * y[e] * x[e];
    const float a = a_c[half];
    const float k = a * a * a * group_sum<16>(sp) / 128.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = a * g[e] * y[e] - x[e] * k;
    *(f32x4*)out = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4*)(out + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
  // RoPE part of head qr: turn the gradient back (transposed rotation), keep
  // it in dQ^ for the gamma reduction, then its RMSNorm backward
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v0 = dr[i >> 1][2 * (i & 1)], v1 = dr[i >> 1][2 * (i & 1) + 1];
    y[2 * i] = v0 * cs[i] + v1 * sn[i];
    y[2 * i + 1] = -v0 * sn[i] + v1 * cs[i];
  }
  *(f32x4*)pr = f32x4{y[0], y[1], y[2], y[3]};
  *(f32x4*)(pr + 4) = f32x4{y[4], y[5], y[6], y[7]};
  float* outr = d_q_rope + qr * 64 + 8 * c8;
  if (!d.qk_norm) {
    *(f32x4*)outr = f32x4{y[0], y[1], y[2], y[3]};
    *(f32x4*)(outr + 4) = f32x4{y[4], y[5], y[6], y[7]};
    return;
  }
  bf16x8_to_f32(xr, x);
  float sp = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) sp += gr[e] * y[e] * x[e];
  const float k = a_r * a_r * a_r * group_sum<8>(sp) / 64.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = a_r * gr[e] * y[e] - x[e] * k;
  *(f32x4*)outr = f32x4{o[0], o[1], o[2], o[3]};
  *(f32x4*)(outr + 4) = f32x4{o[4], o[5], o[6], o[7]};
}

// ---- backward: key norms and the shared RoPE key -------------------------------------
// One workgroup per token row.  Wave w runs the content-key RMSNorm backward
// of groups w, w+4, ...; then the RoPE key gradient is summed over the
// groups (the key is shared by every head), turned back, stored for the
// gamma reduction and taken through its RMSNorm backward.
template <typename T>
__global__ __launch_bounds__(256) void k_norm_bwd_kernel(
    TrainDims d, const T* __restrict__ k_rope, const float* __restrict__ gk,
    const float* __restrict__ gkr, const float* __restrict__ Kraw, const float* __restrict__ ak,
    const float* __restrict__ akr, const float* __restrict__ dKh, float* __restrict__ dK,
    float* __restrict__ dKr, float* __restrict__ d_k_rope) {
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pos = d.rpos[row];
  for (int g = wave; g < d.G; g += 4) {
    const size_t kg = row * d.G + g;
    const float* dy = dKh + kg * d.dqk;
    const float* x = Kraw + kg * d.dc;
    float* out = dK + kg * d.dc;
    if (d.qk_norm)
      rmsnorm_bwd_wave(
          d.dc, ak[kg], gk, [&](int e) { return dy[e]; }, [&](int e) { return x[e]; },
          [&](int e, float v) { out[e] = v; }, lane);
    else
      for (int e = lane; e < d.dc; e += 64) out[e] = dy[e];
  }
  // RoPE key: sum over groups, then the transposed rotation, pair by pair
  float* dyr = dKr + row * d.dr;
  for (int i = tid; i < d.dr / 2; i += 256) {
    float y0 = 0.f, y1 = 0.f;
    for (int g = 0; g < d.G; ++g) {
      const float* src = dKh + (row * d.G + g) * d.dqk + d.dc;
      y0 += src[2 * i];
      y1 += src[2 * i + 1];
    }
    float cs, sn;
    rope_at(d, pos, i, &cs, &sn);
    dyr[2 * i] = y0 * cs + y1 * sn;
    dyr[2 * i + 1] = -y0 * sn + y1 * cs;
  }
  __syncthreads();
  if (wave != 0) return;
  const T* xr = k_rope + row * d.dr;
  float* out = d_k_rope + row * d.dr;
  if (d.qk_norm)
    rmsnorm_bwd_wave(
        d.dr, akr[row], gkr, [&](int e) { return dyr[e]; },
        [&](int e) { return Elem<T>::load(xr, e); }, [&](int e, float v) { out[e] = v; }, lane);
  else
    for (int e = lane; e < d.dr; e += 64) out[e] = dyr[e];
}

// ---- backward: latent gradient --------------------------------------------------------
// d_c_t = sum_g (dk_{t,g} W^UK_g^T + dV_{t,g} W^UV_g^T).  Workgroup = kLatTok
// token rows; thread i owns latent dims i, i + 256, ...
template <typename T>
__global__ __launch_bounds__(256) void latent_bwd_kernel(TrainDims d, int n_rows,
                                                         const float* __restrict__ w_uk,
                                                         const T* __restrict__ w_uv,
                                                         const float* __restrict__ dK,
                                                         const float* __restrict__ dV,
                                                         float* __restrict__ d_c) {
  extern __shared__ float lds[];  // [kLatTok][dc + dv] for one group
  const size_t row0 = (size_t)blockIdx.x * kLatTok;
  const int tid = threadIdx.x;
  const int ntok = (int)min((size_t)kLatTok, (size_t)n_rows - row0);
  const int w = d.dc + d.dv;
  constexpr int kPer = 4;  // r <= 1024
  float acc[kLatTok][kPer];
#pragma unroll
  for (int t = 0; t < kLatTok; ++t)
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[t][k] = 0.f;
  for (int g = 0; g < d.G; ++g) {
    __syncthreads();
    for (int e = tid; e < kLatTok * w; e += 256) {
      const int t = e / w, x = e % w;
      float v = 0.f;
      if (t < ntok)
        v = x < d.dc ? dK[((row0 + t) * d.G + g) * d.dc + x]
                     : dV[((row0 + t) * d.G + g) * d.dv + (x - d.dc)];
      lds[e] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + 256 * k;
      if (i >= d.r) break;
      const float* wk = w_uk + ((size_t)g * d.r + i) * d.dc;
      for (int x = 0; x < d.dc; ++x) {
        const float wv = wk[x];
#pragma unroll
        for (int t = 0; t < kLatTok; ++t) acc[t][k] += lds[t * w + x] * wv;
      }
      const T* wv_row = w_uv + ((size_t)g * d.r + i) * d.dv;
      for (int x = 0; x < d.dv; ++x) {
        const float wv = Elem<T>::load(wv_row, x);
#pragma unroll
        for (int t = 0; t < kLatTok; ++t) acc[t][k] += lds[t * w + d.dc + x] * wv;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = tid + 256 * k;
    if (i >= d.r) break;
#pragma unroll
    for (int t = 0; t < kLatTok; ++t)
      if (t < ntok) d_c[(row0 + t) * d.r + i] = acc[t][k];
  }
}

// ---- backward: up-projection weight gradients -----------------------------------------
// dW_g[i][x] = sum_t c_t[i] dY_{t,g}[x] with dY = dk (W^UK, blockIdx.z = 0) or
// dV (W^UV, blockIdx.z = 1).  Workgroup = kWgRows latent rows of one group;
// thread x owns column x (<= 256).  Deterministic: one sum per output.
template <typename T>
__global__ __launch_bounds__(256) void weight_grad_kernel(TrainDims d, int n_rows,
                                                          const T* __restrict__ c,
                                                          const float* __restrict__ dK,
                                                          const float* __restrict__ dV,
                                                          float* __restrict__ d_w_uk,
                                                          float* __restrict__ d_w_uv) {
  __shared__ float cs[kWgTok][kWgRows];
  __shared__ float ys[kWgTok][256];
  const int i0 = blockIdx.x * kWgRows, g = blockIdx.y, which = blockIdx.z;
  const int D = which == 0 ? d.dc : d.dv;
  const float* Y = which == 0 ? dK : dV;
  const int tid = threadIdx.x;
  float acc[kWgRows];
#pragma unroll
  for (int k = 0; k < kWgRows; ++k) acc[k] = 0.f;
  for (size_t t0 = 0; t0 < (size_t)n_rows; t0 += kWgTok) {
    __syncthreads();
    for (int e = tid; e < kWgTok * kWgRows; e += 256) {
      const int t = e / kWgRows, k = e % kWgRows;
      const bool in = t0 + t < (size_t)n_rows && i0 + k < d.r;
      cs[t][k] = in ? Elem<T>::load(c, (t0 + t) * d.r + i0 + k) : 0.f;
    }
    for (int e = tid; e < kWgTok * D; e += 256) {
      const int t = e / D, x = e % D;
      ys[t][x] = t0 + t < (size_t)n_rows ? Y[((t0 + t) * d.G + g) * D + x] : 0.f;
    }
    __syncthreads();
    if (tid < D) {
      for (int t = 0; t < kWgTok; ++t) {
        const float y = ys[t][tid];
#pragma unroll
        for (int k = 0; k < kWgRows; ++k) acc[k] += cs[t][k] * y;
      }
    }
  }
  if (tid >= D) return;
  float* out = (which == 0 ? d_w_uk : d_w_uv) + (size_t)g * d.r * D;
#pragma unroll
  for (int k = 0; k < kWgRows; ++k)
    if (i0 + k < d.r) out[(size_t)(i0 + k) * D + tid] = acc[k];
}

// ---- backward: RMSNorm weight gradients ------------------------------------------------
// dgamma[x] = sum_rows dy[row][x] x[row][x] a[row]; one partial sum per column
// and row range, then gamma_final_kernel adds them in order.  Block (x, y) takes
// columns 64 x .. 64 x + 63 of the y-th of gridDim.y contiguous row ranges:
// each wave reads 64 consecutive columns of a row (coalesced), the four waves
// interleave rows and meet in LDS.  Every sum has a fixed order.
template <typename X>
__global__ __launch_bounds__(256) void gamma_partial_kernel(int rows, int n, const float* dy,
                                                            int dy_stride, const X* x,
                                                            int x_stride, const float* a,
                                                            float* partial) {
  __shared__ float red[4][64];
  const int c = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + c;
  const int r0 = (int)((int64_t)blockIdx.y * rows / gridDim.y);
  const int r1 = (int)((int64_t)(blockIdx.y + 1) * rows / gridDim.y);
  float s = 0.f;
  if (col < n)
    for (int row = r0 + rl; row < r1; row += 4)
      s += dy[(size_t)row * dy_stride + col] * Elem<X>::load(x, (size_t)row * x_stride + col) *
           a[row];
  red[rl][c] = s;
  __syncthreads();
  if (rl == 0 && col < n)
    partial[(size_t)blockIdx.y * n + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// Block x adds the partials of columns 16 x .. 16 x + 15: lane group k
// (16 groups of 16 threads) takes partials k, k + 16, ..., and the groups meet
// in LDS in a fixed order.
__global__ __launch_bounds__(256) void gamma_final_kernel(int n, int splits, const float* partial,
                                                          float* out, int zero) {
  __shared__ float red[16][16];
  const int c = threadIdx.x & 15, k0 = threadIdx.x >> 4;
  const int col = blockIdx.x * 16 + c;
  float s = 0.f;
  if (!zero && col < n)
#pragma unroll 8
    for (int k = k0; k < splits; k += 16) s += partial[(size_t)k * n + col];
  red[k0][c] = s;
  __syncthreads();
  if (k0 == 0 && col < n) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][c];
    out[col] = t;
  }
}

// ---- MFMA path: keys and values from the GEMM results ------------------------------
// One workgroup per token row: the RMSNorm of each group's raw key (wave per
// group), the normalised, rotated RoPE key (computed once, written into every
// group's row), and the values, all to the bf16 key-major operands.
__global__ __launch_bounds__(256) void kv_norm_kernel(
    TrainDims d, const uint16_t* __restrict__ k_rope, const float* __restrict__ gk,
    const float* __restrict__ gkr, const float* __restrict__ Kraw, const float* __restrict__ V,
    uint16_t* __restrict__ Kb, uint16_t* __restrict__ Vb, float* __restrict__ ak,
    float* __restrict__ akr) {
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = d.rpos[row];
  auto kmaj = [&](int g) { return (size_t)g * d.n_rows + row; };  // group-major rows
  for (int g = wave; g < d.G; g += 4) {
    const float* x = Kraw + (row * d.G + g) * d.dc;
    float a = 1.f;
    if (d.qk_norm) {
      float ss = 0.f;
      for (int e = lane; e < d.dc; e += 64) ss += x[e] * x[e];
      a = 1.0f / sqrtf(wave_sum(ss) / (float)d.dc + d.eps);
      if (lane == 0) ak[row * d.G + g] = a;
    }
    uint16_t* out = Kb + kmaj(g) * d.dqk;
    for (int e = lane; e < d.dc; e += 64) out[e] = f32_to_bf16(x[e] * (d.qk_norm ? gk[e] * a : 1.f));
  }
  for (int e = tid; e < d.G * d.dv; e += 256) {
    const int g = e / d.dv, v = e % d.dv;
    Vb[kmaj(g) * d.dv + v] = f32_to_bf16(V[row * d.G * d.dv + e]);
  }
  if (wave != 0) return;
  const uint16_t* kr = k_rope + row * d.dr;
  float ar = 1.f;
  if (d.qk_norm) {
    float s = 0.f;
    for (int e = lane; e < d.dr; e += 64) {
      const float v = bf16_to_f32(kr[e]);
      s += v * v;
    }
    ar = 1.0f / sqrtf(wave_sum(s) / (float)d.dr + d.eps);
    if (lane == 0) akr[row] = ar;
  }
  for (int i = lane; i < d.dr / 2; i += 64) {
    float x0 = bf16_to_f32(kr[2 * i]), x1 = bf16_to_f32(kr[2 * i + 1]);
    if (d.qk_norm) {
      x0 *= gkr[2 * i] * ar;
      x1 *= gkr[2 * i + 1] * ar;
    }
    float c0, s0;
    rope_at(d, t, i, &c0, &s0);
    const uint16_t y0 = f32_to_bf16(x0 * c0 - x1 * s0), y1 = f32_to_bf16(x0 * s0 + x1 * c0);
    for (int g = 0; g < d.G; ++g) {
      uint16_t* out = Kb + kmaj(g) * d.dqk + d.dc;
      out[2 * i] = y0;
      out[2 * i + 1] = y1;
    }
  }
}

// fp32 -> bf16 (round to nearest even); with `lo`, also the rounding
// remainder in bf16, so that hi + lo carries about 16 bits of the value.
__global__ __launch_bounds__(256) void to_bf16_kernel(size_t n, const float* __restrict__ src,
                                                      uint16_t* __restrict__ hi,
                                                      uint16_t* __restrict__ lo) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint16_t h = f32_to_bf16(src[i]);
    hi[i] = h;
    if (lo) lo[i] = f32_to_bf16(src[i] - bf16_to_f32(h));
  }
}

hipError_t launch_to_bf16(size_t n, const float* src, void* hi, void* lo, hipStream_t s) {
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, s, n, src, (uint16_t*)hi, (uint16_t*)lo);
  return hipGetLastError();
}

}  // namespace

// ---- workspace ------------------------------------------------------------------------
TrainWs train_ws_layout(const Cfg& c, const TrainSeqs& q) {
  const size_t BT = (size_t)q.n_rows, dqk = c.dc + c.dr;
  TrainWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  const bool mf = train_mfma_shape(c);
  w.seqs = take((size_t)q.n_seq * 8);
  w.rpos = take(BT * 4);
  w.rlen = take(BT * 4);
  w.Qh = take(mf ? 0 : BT * c.H * dqk * 4);  // the MFMA path keeps bf16 operands instead
  w.Kh = take(mf ? 0 : BT * c.G * dqk * 4);
  w.V = take(BT * c.G * c.dv * 4);
  w.Kraw = take(BT * c.G * c.dc * 4);
  w.aq = take(BT * c.H * 4);
  w.aqr = take(BT * c.H * 4);
  w.ak = take(BT * c.G * 4);
  w.akr = take(BT * 4);
  w.rope_cs = take((size_t)q.max_len * (c.dr / 2) * 8);
  w.Qb = take(mf ? BT * c.H * dqk * 2 : 0);
  w.Kb = take(mf ? BT * c.G * dqk * 2 : 0);
  w.Vb = take(mf ? BT * c.G * c.dv * 2 : 0);
  w.Wk16 = take(mf ? (size_t)c.G * c.r * c.dc * 2 * 2 : 0);  // bf16 hi, then lo
  w.fwd_total = off;
  w.dQh = take(BT * c.H * dqk * 4);
  w.dKh = take(BT * c.G * dqk * 4);
  w.dV = take(BT * c.G * c.dv * 4);
  w.Dsum = take(BT * c.H * 4);
  w.dK = take(BT * c.G * c.dc * 4);
  w.dKr = take(BT * c.dr * 4);
  w.gamma_partial = take((size_t)kGammaSplit * (c.dc > c.dr ? c.dc : c.dr) * 4);
  w.dOb = take(mf ? BT * c.H * c.dv * 2 : 0);
  w.stat = take(mf ? BT * c.H * 8 : 0);
  w.dKb = take(mf ? BT * c.G * c.dc * 2 : 0);
  w.dVb = take(mf ? BT * c.G * c.dv * 2 : 0);
  const int fbs = mf ? flash_bwd_splits(q.n_seq, q.max_len, c.G) : 1;
  w.fb_part = take(fbs > 1 ? fbs * BT * c.G * (dqk + c.dv) * 4 : 0);
  w.total = off;
  return w;
}

#define WS(type, field) ((type*)(wsb + ws.field))

// Sequence and row tables, RoPE angles; returns the dims every kernel takes.
static TrainDims launch_tables(const Cfg& c, const TrainSeqs& q, const TrainWs& ws, char* wsb,
                               int32_t* status, hipStream_t s) {
  const TrainDims d =
      dims_of(c, q, WS(const float2, rope_cs), WS(const int32_t, rpos), WS(const int32_t, rlen));
  hipLaunchKernelGGL(seq_table_kernel, dim3((q.n_seq + 255) / 256), dim3(256), 0, s, q.n_seq,
                     q.cu, q.n_rows, q.max_len, WS(int2, seqs), status);
  hipLaunchKernelGGL(row_init_kernel, dim3((q.n_rows + 255) / 256), dim3(256), 0, s, q.n_rows,
                     WS(int32_t, rpos), WS(int32_t, rlen));
  hipLaunchKernelGGL(row_fill_kernel, dim3(q.n_seq), dim3(256), 0, s, WS(const int2, seqs),
                     WS(int32_t, rpos), WS(int32_t, rlen));
  const size_t n = (size_t)q.max_len * (d.dr / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     q.max_len, d.dr, d.base, WS(float2, rope_cs));
  return d;
}

// Normalised, rotated queries: fp32 for the row-parallel kernels, or (MF) the
// bf16 operand of the MFMA attention.
template <typename T, bool MF>
static void launch_prep_q(const TrainDims& d, const TrainPtrs& in, const TrainWs& ws, char* wsb,
                          hipStream_t s) {
  if constexpr (MF) {
    if (d.dc == 128 && d.dr == 64 && d.H % kMfHeads == 0 &&
        (((uintptr_t)in.q_c | (uintptr_t)in.q_rope | (uintptr_t)in.gamma_q |
          (uintptr_t)in.gamma_q_rope) & 15) == 0) {
      const dim3 grid(d.n_rows, (d.H + 4 * kMfHeads - 1) / (4 * kMfHeads));
      hipLaunchKernelGGL(prep_q_mf_kernel, grid, dim3(256), 0, s, d, (const uint16_t*)in.q_c,
                         (const uint16_t*)in.q_rope, in.gamma_q, in.gamma_q_rope,
                         WS(uint16_t, Qb), WS(float, aq), WS(float, aqr));
      return;
    }
  }
  hipLaunchKernelGGL((prep_q_kernel<T, MF>), dim3(d.n_rows, (d.H + 3) / 4), dim3(256), 0, s, d,
                     (const T*)in.q_c, (const T*)in.q_rope, in.gamma_q, in.gamma_q_rope,
                     WS(float, Qh), WS(uint16_t, Qb), WS(float, aq), WS(float, aqr));
}

// Row-parallel path: fp32 normalised, rotated queries and keys, values and
// the inverse RMS values.
template <typename T>
static void launch_prep(const TrainDims& d, const TrainPtrs& in, const TrainWs& ws, char* wsb,
                        hipStream_t s) {
  const int n_rows = d.n_rows;
  launch_prep_q<T, false>(d, in, ws, wsb, s);
  hipLaunchKernelGGL((prep_kv_kernel<T>), dim3((n_rows + kKvTok - 1) / kKvTok, d.G), dim3(256),
                     (kKvTok * d.r + kKvTok * 4) * sizeof(float), s, d, n_rows, (const T*)in.c,
                     (const T*)in.k_rope, in.w_uk, (const T*)in.w_uv, in.gamma_k, in.gamma_k_rope,
                     WS(float, Kh), WS(float, Kraw), WS(float, V), WS(float, ak), WS(float, akr));
}

// MFMA path (bf16 layer): Q^ from prep_q; k = c W^UK_g and v = c W^UV_g as
// batched GEMMs (batch = group) into Kraw and V, then kv_norm_kernel forms
// the bf16 group-major operands.
static hipError_t mfma_prep(const TrainDims& d, const TrainPtrs& in, const TrainWs& ws, char* wsb,
                            hipStream_t s) {
  const int BT = d.n_rows;
  launch_prep_q<uint16_t, true>(d, in, ws, wsb, s);
  // W^UK in bf16 hi and lo: c is exact in bf16, so k = c W_hi + c W_lo keeps
  // the key (and its RMS) close to fp32
  const size_t nw = (size_t)d.G * d.r * d.dc;
  const uint16_t* w_hi = WS(const uint16_t, Wk16);
  hipError_t e = launch_to_bf16(nw, in.w_uk, wsb + ws.Wk16, wsb + ws.Wk16 + nw * 2, s);
  if (e != hipSuccess) return e;
  const GemmOperand A{(const uint16_t*)in.c, d.r, 1 << 30, 0, 0};  // c [BT][r], K-contiguous
  GemmArgs g{A, GemmOperand{w_hi, d.dc, 1 << 30, 0, (int64_t)d.r * d.dc}, WS(float, Kraw),
             (int64_t)d.G * d.dc, d.dc, BT, d.dc, d.r, 0};
  if ((e = launch_gemm_bf16(g, true, false, d.G, s)) != hipSuccess) return e;
  g.B.p = w_hi + nw;
  g.accumulate = 1;
  if ((e = launch_gemm_bf16(g, true, false, d.G, s)) != hipSuccess) return e;
  g.accumulate = 0;
  g.B = GemmOperand{(const uint16_t*)in.w_uv, d.dv, 1 << 30, 0, (int64_t)d.r * d.dv};
  g.C = WS(float, V);
  g.ldc = (int64_t)d.G * d.dv;
  g.c_batch_stride = d.dv;
  g.N = d.dv;
  if ((e = launch_gemm_bf16(g, true, false, d.G, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(kv_norm_kernel, dim3(BT), dim3(256), 0, s, d, (const uint16_t*)in.k_rope,
                     in.gamma_k, in.gamma_k_rope, WS(const float, Kraw), WS(const float, V),
                     WS(uint16_t, Kb), WS(uint16_t, Vb), WS(float, ak), WS(float, akr));
  return hipGetLastError();
}

// MFMA path: dc = dk W^UK^T + dV W^UV^T (K runs over (group, dim)) and
// dW_g = c^T dY_g, from bf16 copies of dk and dV.
static hipError_t mfma_projection_grads(const TrainDims& d, const TrainPtrs& in,
                                        const TrainWs& ws, char* wsb, const TrainGrads& gr,
                                        hipStream_t s) {
  const int BT = d.n_rows;
  hipError_t e =
      launch_to_bf16((size_t)BT * d.G * d.dc, WS(const float, dK), wsb + ws.dKb, nullptr, s);
  if (e != hipSuccess) return e;
  if ((e = launch_to_bf16((size_t)BT * d.G * d.dv, WS(const float, dV), wsb + ws.dVb, nullptr,
                          s)) != hipSuccess)
    return e;
  // latent gradient: A = dk [BT][G*dc] (K-contiguous), B(k=(g,j), n=i) = W^UK[g][i][j]
  GemmArgs g{GemmOperand{WS(const uint16_t, dKb), (int64_t)d.G * d.dc, 1 << 30, 0, 0},
             GemmOperand{WS(const uint16_t, Wk16), d.dc, d.dc, (int64_t)d.r * d.dc, 0},
             gr.d_c, d.r, 0, BT, d.r, d.G * d.dc, 0};
  if ((e = launch_gemm_bf16(g, true, true, 1, s)) != hipSuccess) return e;
  g.A = GemmOperand{WS(const uint16_t, dVb), (int64_t)d.G * d.dv, 1 << 30, 0, 0};
  g.B = GemmOperand{(const uint16_t*)in.w_uv, d.dv, d.dv, (int64_t)d.r * d.dv, 0};
  g.K = d.G * d.dv;
  g.accumulate = 1;
  if ((e = launch_gemm_bf16(g, true, true, 1, s)) != hipSuccess) return e;
  // weight gradients, batch = group: A(m=i, k=t) = c[t][i], B(k=t, n=j) = dk[t][g][j]
  GemmArgs w{GemmOperand{(const uint16_t*)in.c, d.r, 1 << 30, 0, 0},
             GemmOperand{WS(const uint16_t, dKb), (int64_t)d.G * d.dc, 1 << 30, 0, d.dc},
             gr.d_w_uk, d.dc, (int64_t)d.r * d.dc, d.r, d.dc, BT, 0};
  if ((e = launch_gemm_bf16(w, false, false, d.G, s)) != hipSuccess) return e;
  w.B = GemmOperand{WS(const uint16_t, dVb), (int64_t)d.G * d.dv, 1 << 30, 0, d.dv};
  w.C = gr.d_w_uv;
  w.ldc = d.dv;
  w.c_batch_stride = (int64_t)d.r * d.dv;
  w.N = d.dv;
  return launch_gemm_bf16(w, false, false, d.G, s);
}

static FlashSeqs flash_seqs(const TrainDims& d, const TrainWs& ws, char* wsb) {
  return FlashSeqs{d.n_rows, d.n_seq, d.max_len, WS(const int2, seqs)};
}

template <typename T>
static hipError_t forward_impl(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                               const TrainWs& ws, char* wsb, float* o, float* lse,
                               int32_t* status, hipStream_t s) {
  const TrainDims d = launch_tables(c, q, ws, wsb, status, s);
  if (train_mfma_shape(c)) {
    const hipError_t e = mfma_prep(d, in, ws, wsb, s);
    if (e != hipSuccess) return e;
    return launch_flash_fwd(c, flash_seqs(d, ws, wsb), wsb + ws.Qb, wsb + ws.Kb, wsb + ws.Vb, o,
                            lse, s);
  }
  launch_prep<T>(d, in, ws, wsb, s);
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(d.n_rows, d.H), dim3(256),
                     (d.dqk + kChunk + 4) * sizeof(float), s, d, WS(const float, Qh),
                     WS(const float, Kh), WS(const float, V), o, lse);
  return hipGetLastError();
}

template <typename T>
static hipError_t backward_impl(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                                const float* o, const float* lse, const float* d_o,
                                const TrainWs& ws, char* wsb, const TrainGrads& gr,
                                int32_t* status, hipStream_t s) {
  const TrainDims d = launch_tables(c, q, ws, wsb, status, s);
  const int n_rows = d.n_rows;
  const bool mf = train_mfma_shape(c);
  if (mf) {
    hipError_t e = mfma_prep(d, in, ws, wsb, s);
    if (e != hipSuccess) return e;
    e = launch_flash_bwd(c, flash_seqs(d, ws, wsb), wsb + ws.Qb, wsb + ws.Kb, wsb + ws.Vb, o,
                         lse, d_o, wsb + ws.dOb, wsb + ws.stat, WS(float, dKh), WS(float, dV),
                         WS(float, dQh), WS(float, fb_part), s);
    if (e != hipSuccess) return e;
  } else {
    launch_prep<T>(d, in, ws, wsb, s);
    hipLaunchKernelGGL(attn_bwd_q_kernel, dim3(n_rows, d.H), dim3(256),
                       (d.dqk + d.dv + kChunk + 4) * sizeof(float), s, d, WS(const float, Qh),
                       WS(const float, Kh), WS(const float, V), o, lse, d_o, WS(float, dQh),
                       WS(float, Dsum));
    hipLaunchKernelGGL(attn_bwd_kv_kernel, dim3(n_rows, d.G), dim3(256),
                       (d.dqk + d.dv + 2 * kChunk) * sizeof(float), s, d, WS(const float, Qh),
                       WS(const float, Kh), WS(const float, V), lse, d_o, WS(const float, Dsum),
                       WS(float, dKh), WS(float, dV));
  }
  if (mf && d.dc == 128 && d.dr == 64 && d.H % kMfHeads == 0 &&
      (((uintptr_t)in.q_c | (uintptr_t)in.q_rope | (uintptr_t)in.gamma_q |
        (uintptr_t)in.gamma_q_rope | (uintptr_t)gr.d_q_c | (uintptr_t)gr.d_q_rope) & 15) == 0)
    hipLaunchKernelGGL(q_norm_bwd_mf_kernel,
                       dim3(n_rows, (d.H + 4 * kMfHeads - 1) / (4 * kMfHeads)), dim3(256), 0, s, d,
                       (const uint16_t*)in.q_c, (const uint16_t*)in.q_rope, in.gamma_q,
                       in.gamma_q_rope, WS(const float, aq), WS(const float, aqr), WS(float, dQh),
                       gr.d_q_c, gr.d_q_rope);
  else
    hipLaunchKernelGGL(q_norm_bwd_kernel<T>, dim3(n_rows, (d.H + 3) / 4), dim3(256), 0, s, d,
                       (const T*)in.q_c, (const T*)in.q_rope, in.gamma_q, in.gamma_q_rope,
                       WS(const float, aq), WS(const float, aqr), WS(float, dQh), gr.d_q_c,
                       gr.d_q_rope);
  hipLaunchKernelGGL(k_norm_bwd_kernel<T>, dim3(n_rows), dim3(256), 0, s, d, (const T*)in.k_rope,
                     in.gamma_k, in.gamma_k_rope, WS(const float, Kraw), WS(const float, ak),
                     WS(const float, akr), WS(const float, dKh), WS(float, dK), WS(float, dKr),
                     gr.d_k_rope);
  if (mf) {
    const hipError_t e = mfma_projection_grads(d, in, ws, wsb, gr, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(latent_bwd_kernel<T>, dim3((n_rows + kLatTok - 1) / kLatTok), dim3(256),
                       (size_t)kLatTok * (d.dc + d.dv) * sizeof(float), s, d, n_rows, in.w_uk,
                       (const T*)in.w_uv, WS(const float, dK), WS(const float, dV), gr.d_c);
    hipLaunchKernelGGL(weight_grad_kernel<T>, dim3((d.r + kWgRows - 1) / kWgRows, d.G, 2),
                       dim3(256), 0, s, d, n_rows, (const T*)in.c, WS(const float, dK),
                       WS(const float, dV), gr.d_w_uk, gr.d_w_uv);
  }
  // RMSNorm weights: (dy, x, a) per gamma; all zero in plain mode
  float* part = WS(float, gamma_partial);
  struct G4 {
    int rows, n;
    const float* dy;
    int dys;
    const void* x;
    int xs;
    bool x_f32;
    const float* a;
    float* out;
  } gs[4] = {
      {n_rows * d.H, d.dc, WS(const float, dQh), d.dqk, in.q_c, d.dc, false, WS(const float, aq),
       gr.d_gamma_q},
      {n_rows * d.G, d.dc, WS(const float, dKh), d.dqk, WS(const float, Kraw), d.dc, true,
       WS(const float, ak), gr.d_gamma_k},
      {n_rows * d.H, d.dr, WS(const float, dQh) + d.dc, d.dqk, in.q_rope, d.dr, false,
       WS(const float, aqr), gr.d_gamma_q_rope},
      {n_rows, d.dr, WS(const float, dKr), d.dr, in.k_rope, d.dr, false, WS(const float, akr),
       gr.d_gamma_k_rope},
  };
  for (const G4& q : gs) {
    const int splits = gamma_splits(q.rows);
    const dim3 grid((q.n + 63) / 64, splits);
    if (d.qk_norm) {
      if (q.x_f32)
        hipLaunchKernelGGL(gamma_partial_kernel<float>, grid, dim3(256), 0, s, q.rows, q.n, q.dy,
                           q.dys, (const float*)q.x, q.xs, q.a, part);
      else
        hipLaunchKernelGGL(gamma_partial_kernel<T>, grid, dim3(256), 0, s, q.rows, q.n, q.dy,
                           q.dys, (const T*)q.x, q.xs, q.a, part);
    }
    hipLaunchKernelGGL(gamma_final_kernel, dim3((q.n + 15) / 16), dim3(256), 0, s, q.n, splits,
                       part, q.out, d.qk_norm ? 0 : 1);
  }
  return hipGetLastError();
}

hipError_t launch_train_forward(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                                const TrainWs& ws, void* workspace, float* o, float* lse,
                                int32_t* status, hipStream_t s) {
  char* wsb = (char*)workspace;
  return c.dtype == QKMLA_BF16
             ? forward_impl<uint16_t>(c, q, in, ws, wsb, o, lse, status, s)
             : forward_impl<float>(c, q, in, ws, wsb, o, lse, status, s);
}

hipError_t launch_train_backward(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                                 const float* o, const float* lse, const float* d_o,
                                 const TrainWs& ws, void* workspace, const TrainGrads& gr,
                                 int32_t* status, hipStream_t s) {
  char* wsb = (char*)workspace;
  return c.dtype == QKMLA_BF16
             ? backward_impl<uint16_t>(c, q, in, o, lse, d_o, ws, wsb, gr, status, s)
             : backward_impl<float>(c, q, in, o, lse, d_o, ws, wsb, gr, status, s);
}

}  // namespace qkmla
