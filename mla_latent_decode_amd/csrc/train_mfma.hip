// Causal attention forward of the training / prefill path on gfx950 MFMA, for
// the bf16 layer with 16 query heads per KV group, d_c + d_r = 192 and
// d_v = 128 ("QK-Normed MLA: QK normalization without full key caching",
// technical summary, Methodology: Blockwise Normalization; the content and
// RoPE parts of each normalised query and key sit side by side, so one
// 192-dim dot product gives the whole logit).
//
// Workgroup = (sequence s, group g, block of 8 query tokens); wave w owns 32
// query rows = tokens 2w, 2w+1 of the block x the group's 16 heads, so all
// four waves share every 32-key tile of K^ and V.  Per key tile:
//   S^T (32 keys x 32 rows) = K^ (32 x 192) . Q^T      (12 MFMA 32x32x16)
//   online softmax per row (exp2 domain: Q^ carries tau*log2(e))
//   O^T (128 dims x 32 rows) += V^T (128 x 32) . P^T  (8 MFMA 32x32x16)
// With S^T (keys as rows) each lane holds one query row, so the row max and
// sum are in-lane plus one exchange with the other half of the wavefront.
// MFMA 32x32x16 bf16 layouts: A lane l holds A[m=l%32][k=8(l/32)+j]; B lane l
// holds B[k=8(l/32)+j][n=l%32]; D lane l reg i holds D[8(i/4)+4(l/32)+i%4][l%32].
// P^T goes from the S^T accumulator straight into the B operand of P.V; its
// key order is matched by reading V^T with ds_read_b64_tr_b16 (within each
// 16-lane group lane i receives element i%4 of the 8-byte loads of lanes
// 4e + i/4), which turns 4 key rows into 4 keys of one dim.
//
// K^ and V tiles are loaded to registers one tile ahead and written to a
// double-buffered, padded LDS stage: one barrier per tile.  The forward fits
// in 256 registers without spills, so two workgroups share a CU (two waves
// per SIMD hide each other's tile loads).
#include "device_common.h"
#include "qkmla_internal.h"

namespace qkmla {

namespace {

constexpr int kFaKeys = 32;                 // keys per tile
constexpr int kFaTok = 8;                   // query tokens per workgroup
constexpr int kFaHpg = 16;                  // heads per group
constexpr int kFaDqk = 192;                 // d_c + d_r
constexpr int kFaDv = 128;                  // d_v
constexpr int kKPitch = kFaDqk * 2 + 16;    // 400 B per key row in LDS
constexpr int kVPitch = kFaDv * 2 + 16;     // 272 B per value row in LDS
constexpr int kKChunks = kFaKeys * kFaDqk * 2 / 16;  // 768 16-byte chunks per K tile
constexpr int kVChunks = kFaKeys * kFaDv * 2 / 16;   // 512 per V tile
constexpr int kQkSteps = kFaDqk / 16;       // 12
constexpr int kDvBlocks = kFaDv / 32;       // 4
// Key side of the backward: each 128-key block's causal token range is cut
// into up to kFbMaxSplits pieces, as many as bring the grid to about
// kFbTargetWgs workgroups (two per CU).
constexpr int kFbMaxSplits = 8;
constexpr int kFbTargetWgs = 512;

// Token rows are packed: sequence s holds rows seqs[s].x .. + seqs[s].y - 1.
struct FaArgs {
  const uint16_t* Qb;  // [rows][H][192] bf16, scaled by tau*log2(e)
  const uint16_t* Kb;  // [G][rows][192] bf16
  const uint16_t* Vb;  // [G][rows][128] bf16
  float* o;            // [rows][H][128]
  float* lse;          // [rows][H], natural log
  const int2* seqs;    // [n_seq] (start row, length)
  int n_rows, H, G;
};

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *(const uint4*)p;
}

// One 32-key tile of K^ and V: 768 + 512 chunks of 16 B, 3 + 2 per thread of a
// 256-thread workgroup, loaded to registers and stored to a padded LDS stage.
// Keys past the sequence repeat its last key (the callers mask them).
struct KvStage {
  uint4 kr[kKChunks / 256], vr[kVChunks / 256];
  __device__ void load(const uint16_t* kbase, const uint16_t* vbase, int kt, int T, int tid) {
#pragma unroll
    for (int u = 0; u < kKChunks / 256; ++u) {
      const int c = tid + 256 * u, row = c / 24, col = c % 24;
      kr[u] = load16(kbase + (size_t)min(kt * kFaKeys + row, T - 1) * kFaDqk + col * 8);
    }
#pragma unroll
    for (int u = 0; u < kVChunks / 256; ++u) {
      const int c = tid + 256 * u, row = c / 16, col = c % 16;
      vr[u] = load16(vbase + (size_t)min(kt * kFaKeys + row, T - 1) * kFaDv + col * 8);
    }
  }
  __device__ void store(char* k_st, char* v_st, int tid) const {
#pragma unroll
    for (int u = 0; u < kKChunks / 256; ++u) {
      const int c = tid + 256 * u, row = c / 24, col = c % 24;
      *(uint4*)(k_st + row * kKPitch + col * 16) = kr[u];
    }
#pragma unroll
    for (int u = 0; u < kVChunks / 256; ++u) {
      const int c = tid + 256 * u, row = c / 16, col = c % 16;
      *(uint4*)(v_st + row * kVPitch + col * 16) = vr[u];
    }
  }
};

__global__ __launch_bounds__(256, 2) void flash_fwd_kernel(FaArgs a) {
  __shared__ __attribute__((aligned(16))) char k_st[2][kFaKeys * kKPitch];
  __shared__ __attribute__((aligned(16))) char v_st[2][kFaKeys * kVPitch];
  // blockIdx.x = (last query block - qb) * G + g: the blocks with the most
  // key tiles are dispatched first
  const unsigned bx = blockIdx.x, gn = a.G;
  const int qb = (int)(gridDim.x / gn - 1 - bx / gn), g = (int)(bx % gn);
  const int2 sq = a.seqs[blockIdx.z];  // (start row, length), uniform
  const int T = sq.y;
  if (qb * kFaTok >= T) return;  // whole workgroup: past this sequence
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, n = lane & 31;
  const int i = qb * kFaTok + 2 * wave + (n >> 4);  // query token of this lane's column
  const int h = g * kFaHpg + (n & 15);
  const bool valid = i < T;
  const size_t qrow = ((size_t)sq.x + (valid ? i : T - 1)) * a.H + h;

  // Q^T as the B operand of the QK MFMAs, for the whole key loop
  bf16x8 q[kQkSteps];
  {
    const uint16_t* qp = a.Qb + qrow * kFaDqk + 8 * hf;
#pragma unroll
    for (int s = 0; s < kQkSteps; ++s) {
      const uint4 v = load16(qp + 16 * s);
      q[s] = *(const bf16x8*)&v;
    }
  }

  const int i_last = min(qb * kFaTok + kFaTok - 1, T - 1);
  const int n_kt = i_last / kFaKeys + 1;  // key tiles 0 .. i_last / 32 (all 8 tokens in one)
  const uint16_t* kbase = a.Kb + ((size_t)g * a.n_rows + sq.x) * kFaDqk;
  const uint16_t* vbase = a.Vb + ((size_t)g * a.n_rows + sq.x) * kFaDv;

  KvStage stage;
  f32x16 O[kDvBlocks];
#pragma unroll
  for (int mb = 0; mb < kDvBlocks; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Tile kt + 1 waits in registers while tile kt is computed, and tile
  // kt + 2 is on its way: two tiles of load latency hidden.
  KvStage sb;
  stage.load(kbase, vbase, 0, T, tid);
  stage.store(k_st[0], v_st[0], tid);
  if (1 < n_kt) stage.load(kbase, vbase, 1, T, tid);
  __syncthreads();
  auto tile = [&](int kt, int buf, KvStage& next, KvStage& after) {
    if (kt + 2 < n_kt) after.load(kbase, vbase, kt + 2, T, tid);
    const char* ks = k_st[buf];
    const char* vs = v_st[buf];

    // ---- S^T[32 keys][32 rows] ----
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    const char* arow = ks + n * kKPitch + 16 * hf;
#pragma unroll
    for (int s = 0; s < kQkSteps; ++s) {
      const bf16x8 av = *(const bf16x8*)(arow + 32 * s);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, q[s], sacc, 0, 0, 0);
    }

    // ---- causal mask, online softmax (reg r holds key 8(r/4) + 4hf + r%4) ----
    const int key0 = kt * kFaKeys + 4 * hf;
    float lg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) lg[r] = sacc[r];
    // only a tile reaching past the wave's first token (or the sequence) masks
    if (kt * kFaKeys + kFaKeys - 1 > qb * kFaTok + 2 * wave) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + (r & 3);
        if (key > i || key >= T) lg[r] = -INFINITY;
      }
    }
    float mt = lg[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, lg[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);  // finite: key kt*32 <= i for a valid row
    const float f = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(lg[r] - m_new);
    // l sums the weights as rounded for P.V
    float ls = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t* u = (const uint32_t*)&pb[k];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        ls += __uint_as_float(u[d] << 16) + __uint_as_float(u[d] & 0xFFFF0000u);
    }
    l_run = l_run * f + ls;
    if (__ballot(f != 1.0f) != 0) {  // some row's max moved: rescale its O
#pragma unroll
      for (int mb = 0; mb < kDvBlocks; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[mb][r] *= f;
    }

    // ---- O^T[128 dims][32 rows] += V^T . P^T ----
    const int s16 = lane & 15, dblk = (lane >> 4) & 1;
    const char* pvb = vs + (4 * hf + (s16 >> 2)) * kVPitch + 32 * dblk + 8 * (s16 & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mb = 0; mb < kDvBlocks; ++mb) {
        const char* pa = pvb + 16 * kk * kVPitch + 64 * mb;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa + 8 * kVPitch));
        const bf16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, pb[kk], O[mb], 0, 0, 0);
      }
    }
    if (kt + 1 < n_kt) next.store(k_st[buf ^ 1], v_st[buf ^ 1], tid);
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile(kt, 0, stage, sb);
    if (kt + 1 >= n_kt) break;
    tile(kt + 1, 1, sb, stage);
  }

  // ---- epilogue: lane holds O^T[32mb + 8(r/4) + 4hf + r%4][its row] ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!valid) return;
  const float inv = 1.0f / l_tot;
  float* op = a.o + qrow * kFaDv + 4 * hf;
#pragma unroll
  for (int mb = 0; mb < kDvBlocks; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = O[mb][4 * r4 + c] * inv;
      *(f32x4*)(op + 32 * mb + 8 * r4) = v;
    }
  if (hf == 0) a.lse[qrow] = (m_run + log2f(l_tot)) * kLn2;
}

// ---- backward ------------------------------------------------------------------
// Per row (token i, head h): lse2 = lse*log2(e), D = d_o . o, and d_o in bf16.
// One wavefront per (token row, 4 heads) ... one lane per 2 dims.
__global__ __launch_bounds__(256) void bwd_prep_kernel(int n_rows_h, const float* __restrict__ o,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ d_o,
                                                       uint16_t* __restrict__ dOb,
                                                       float2* __restrict__ stat) {
  const size_t rh = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rh >= (size_t)n_rows_h) return;
  const float2 g = *(const float2*)(d_o + rh * kFaDv + 2 * lane);
  const float2 v = *(const float2*)(o + rh * kFaDv + 2 * lane);
  const float D = wave_sum(g.x * v.x + g.y * v.y);
  const uint32_t packed = (uint32_t)f32_to_bf16(g.x) | ((uint32_t)f32_to_bf16(g.y) << 16);
  *(uint32_t*)(dOb + rh * kFaDv + 2 * lane) = packed;
  if (lane == 0) stat[rh] = make_float2(lse[rh] * kLog2e, D);
}

struct FbArgs {
  const uint16_t* Qb;   // [rows][H][192] bf16, scaled by tau*log2(e)
  const uint16_t* Kb;   // [G][rows][192]
  const uint16_t* Vb;   // [G][rows][128]
  const uint16_t* dOb;  // [rows][H][128] bf16
  const float2* stat;   // [rows][H]: (lse*log2(e), D)
  float* dKh;           // [rows][G][192] fp32: dK^ (content | RoPE)
  float* dV;            // [rows][G][128] fp32
  float* dQh;           // [rows][H][192] fp32: dQ^
  const int2* seqs;     // [n_seq] (start row, length)
  int n_rows, H, G;
  float tau;
  // Key side split over `splits` token ranges: range c writes its dK^ / dV
  // into dKp + c [rows][G][192] / dVp + c [rows][G][128] (dKh / dV when 1).
  float* dKp;
  float* dVp;
  int splits;
};

// Key side: workgroup = (sequence, group, 128 keys, token range); wave w
// owns the block's w-th 32-key tile, whose K^ and V stay in its registers as
// B operands.  All four waves share the query rows, which stream through a
// double-buffered LDS stage two tokens (x 16 heads = 32 rows) at a time over
// the workgroup's share of the tokens from the block's first key on; the
// next two steps' rows are in flight during each step.
//   S  (rows x keys) = Q^ . K^T,  dP = d_o . V^T       (lane = key, regs = rows)
//   p = 2^(S - lse2) (0 where key > token), dS = p (dP - D)
//   dV^T (128 x keys) += d_o^T . P,   dK^T (192 x keys) += Q^T . dS
// with d_o^T and Q^T read by ds_read_b64_tr_b16 in the row order of P's regs.
// A wave skips the MFMAs of steps that lie wholly before its keys.
struct RowStage {  // 32 rows: Q^ 768 + d_o 512 chunks of 16 B, 3 + 2 per thread
  uint4 q[3], o[2];
  float2 st;
  __device__ void load(const FbArgs& a, size_t seq_row0, int T, int g, int i0, int tid) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int c = tid + 256 * u, row = c / 24, col = c % 24;
      const int tok = min(i0 + (row >> 4), T - 1);
      const size_t qr = (seq_row0 + tok) * a.H + g * kFaHpg + (row & 15);
      q[u] = load16(a.Qb + qr * kFaDqk + col * 8);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c / 16, col = c % 16;
      const int tok = min(i0 + (row >> 4), T - 1);
      const size_t qr = (seq_row0 + tok) * a.H + g * kFaHpg + (row & 15);
      o[u] = load16(a.dOb + qr * kFaDv + col * 8);
    }
    if (tid < 32) {
      const int tok = min(i0 + (tid >> 4), T - 1);
      st = a.stat[(seq_row0 + tok) * a.H + g * kFaHpg + (tid & 15)];
    }
  }
  __device__ void store(char* q_st, char* o_st, float2* st_s, int tid) const {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int c = tid + 256 * u, row = c / 24, col = c % 24;
      *(uint4*)(q_st + row * kKPitch + col * 16) = q[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u, row = c / 16, col = c % 16;
      *(uint4*)(o_st + row * kVPitch + col * 16) = o[u];
    }
    if (tid < 32) st_s[tid] = st;
  }
};

__global__ __launch_bounds__(256) void flash_bwd_kv_kernel(FbArgs a) {
  __shared__ __attribute__((aligned(16))) char q_st[2][32 * kKPitch];
  __shared__ __attribute__((aligned(16))) char o_st[2][32 * kVPitch];
  __shared__ float2 st_s[2][32];
  // blockIdx.x = (key block * G + g) * splits + split: the longest token
  // ranges (the first key blocks) are dispatched first
  const unsigned bx = blockIdx.x, sp = a.splits, gn = a.G;
  const int split = (int)(bx % sp);  // which token range of the key block
  const int g = (int)(bx / sp % gn);
  const int2 sq = a.seqs[blockIdx.z];  // (start row, length), uniform
  const int T = sq.y;
  const int kblk0 = (int)(bx / (sp * gn)) * 4 * kFaKeys;  // first key of the workgroup
  if (kblk0 >= T) return;  // whole workgroup: past this sequence
  // The key block's tokens kblk0 .. T-1 form n2 two-token steps; this
  // workgroup takes steps [n2 split / splits, n2 (split + 1) / splits).
  const int n2 = (T - kblk0 + 1) / 2;
  const int i_lo = kblk0 + 2 * (int)((int64_t)n2 * split / a.splits);
  const int i_hi = kblk0 + 2 * (int)((int64_t)n2 * (split + 1) / a.splits);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, n = lane & 31;
  const int key0 = kblk0 + wave * kFaKeys;
  const int key = key0 + n;
  const int keyc = min(key, T - 1);
  const size_t kv_row = (size_t)g * a.n_rows + sq.x + keyc;
  bf16x8 kreg[kQkSteps], vreg[kFaDv / 16];
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) {
    const uint4 v = load16(a.Kb + kv_row * kFaDqk + 16 * s + 8 * hf);
    kreg[s] = *(const bf16x8*)&v;
  }
#pragma unroll
  for (int s = 0; s < kFaDv / 16; ++s) {
    const uint4 v = load16(a.Vb + kv_row * kFaDv + 16 * s + 8 * hf);
    vreg[s] = *(const bf16x8*)&v;
  }
  f32x16 dKT[kFaDqk / 32], dVT[kDvBlocks];
#pragma unroll
  for (int mb = 0; mb < kFaDqk / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dKT[mb][r] = 0.f;
#pragma unroll
  for (int mb = 0; mb < kDvBlocks; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dVT[mb][r] = 0.f;

  const size_t seq_row0 = sq.x;
  const int s16 = lane & 15, dblk = (lane >> 4) & 1;
  // Rows of step i0 + 2 wait in registers while step i0 is computed, and
  // those of step i0 + 4 are on their way: two steps of load latency hidden.
  RowStage ra, rb;
  ra.load(a, seq_row0, T, g, i_lo, tid);
  ra.store(q_st[0], o_st[0], st_s[0], tid);
  if (i_lo + 2 < i_hi) ra.load(a, seq_row0, T, g, i_lo + 2, tid);
  __syncthreads();
  auto step = [&](int i0, int buf, RowStage& next, RowStage& after) {
    if (i0 + 4 < i_hi) after.load(a, seq_row0, T, g, i0 + 4, tid);
    // wave-uniform: the step's tokens all precede this wave's keys
    if (i0 + 1 >= key0 && key0 < T) {
      const char* qs = q_st[buf];
      const char* os = o_st[buf];
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.f;
        dpacc[r] = 0.f;
      }
      const char* qrow = qs + n * kKPitch + 16 * hf;
#pragma unroll
      for (int s = 0; s < kQkSteps; ++s)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qrow + 32 * s), kreg[s],
                                                       sacc, 0, 0, 0);
      const char* orow = os + n * kVPitch + 16 * hf;
#pragma unroll
      for (int s = 0; s < kFaDv / 16; ++s)
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(orow + 32 * s), vreg[s],
                                                        dpacc, 0, 0, 0);
      // reg r holds row 8(r/4) + 4hf + r%4 = token i0 + row/16, head row%16; only
      // steps whose tokens can precede a key of the tile, or run past the
      // sequence, or a tile past the sequence, mask (wave-uniform)
      const bool masked = i0 < key0 + kFaKeys - 1 || i0 + 1 >= T || key0 + kFaKeys > T;
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
        const int tok = i0 + (row >> 4);
        const float2 sd = st_s[buf][row];
        float p = __builtin_amdgcn_exp2f(sacc[r] - sd.x);
        if (masked && !(key <= tok && tok < T && key < T)) p = 0.f;
        pb[r >> 3][r & 7] = (__bf16)p;
        db[r >> 3][r & 7] = (__bf16)(p * (dpacc[r] - sd.y));
      }
      const char* tvb = os + (4 * hf + (s16 >> 2)) * kVPitch + 32 * dblk + 8 * (s16 & 3);
      const char* tqb = qs + (4 * hf + (s16 >> 2)) * kKPitch + 32 * dblk + 8 * (s16 & 3);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mb = 0; mb < kDvBlocks; ++mb) {
          const char* pa = tvb + 16 * kk * kVPitch + 64 * mb;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa));
          const bf16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa + 8 * kVPitch));
          const bf16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          dVT[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, pb[kk], dVT[mb], 0, 0, 0);
        }
#pragma unroll
        for (int mb = 0; mb < kFaDqk / 32; ++mb) {
          const char* pa = tqb + 16 * kk * kKPitch + 64 * mb;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa));
          const bf16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa + 8 * kKPitch));
          const bf16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          dKT[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, db[kk], dKT[mb], 0, 0, 0);
        }
      }
    }
    if (i0 + 2 < i_hi) next.store(q_st[buf ^ 1], o_st[buf ^ 1], st_s[buf ^ 1], tid);
    __syncthreads();
  };
  for (int i0 = i_lo; i0 < i_hi; i0 += 4) {
    step(i0, 0, ra, rb);
    if (i0 + 2 >= i_hi) break;
    step(i0 + 2, 1, rb, ra);
  }
  if (key >= T) return;  // (an empty token range still writes its zeros)
  // lane holds column `key`; reg r of block mb is dim 32mb + 8(r/4) + 4hf + r%4.
  // Q^ carries tau*log2(e): dK^ = tau sum dS Q^ = (sum dS Qb) / log2(e).
  const size_t out_row = (size_t)split * a.n_rows * a.G + (seq_row0 + key) * a.G + g;
  float* dk = a.dKp + out_row * kFaDqk + 4 * hf;
  float* dv = a.dVp + out_row * kFaDv + 4 * hf;
#pragma unroll
  for (int mb = 0; mb < kFaDqk / 32; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = dKT[mb][4 * r4 + c] * kLn2;
      *(f32x4*)(dk + 32 * mb + 8 * r4) = v;
    }
#pragma unroll
  for (int mb = 0; mb < kDvBlocks; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = dVT[mb][4 * r4 + c];
      *(f32x4*)(dv + 32 * mb + 8 * r4) = v;
    }
}

// out[i] = sum over the splits c of part[c n4 + i], in order of c.
__global__ __launch_bounds__(256) void split_sum_kernel(size_t n4, int splits,
                                                        const f32x4* __restrict__ part,
                                                        f32x4* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = part[i];
  for (int c = 1; c < splits; ++c) acc += part[(size_t)c * n4 + i];
  out[i] = acc;
}

// Query side: the forward's workgroup shape (8 tokens x 16 heads, four
// wavefronts sharing each 32-key tile).  Per key tile:
//   S^T = K^ . Q^T,  dP^T = V . d_o^T                  (lane = row, regs = keys)
//   dS^T = 2^(S^T - lse2) (dP^T - D),  dQ^T (192 x rows) += K^T . dS^T
// with K^T read by ds_read_b64_tr_b16 in the key order of dS's regs.
__global__ __launch_bounds__(256) void flash_bwd_q_kernel(FbArgs a) {
  __shared__ __attribute__((aligned(16))) char k_st[2][kFaKeys * kKPitch];
  __shared__ __attribute__((aligned(16))) char v_st[2][kFaKeys * kVPitch];
  // blockIdx.x = (last query block - qb) * G + g: the blocks with the most
  // key tiles are dispatched first
  const unsigned bx = blockIdx.x, gn = a.G;
  const int qb = (int)(gridDim.x / gn - 1 - bx / gn), g = (int)(bx % gn);
  const int2 sq = a.seqs[blockIdx.z];  // (start row, length), uniform
  const int T = sq.y;
  if (qb * kFaTok >= T) return;  // whole workgroup: past this sequence
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, n = lane & 31;
  const int i = qb * kFaTok + 2 * wave + (n >> 4);
  const int h = g * kFaHpg + (n & 15);
  const bool valid = i < T;
  const size_t qrow = ((size_t)sq.x + (valid ? i : T - 1)) * a.H + h;
  bf16x8 q[kQkSteps], go[kFaDv / 16];
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) {
    const uint4 v = load16(a.Qb + qrow * kFaDqk + 16 * s + 8 * hf);
    q[s] = *(const bf16x8*)&v;
  }
#pragma unroll
  for (int s = 0; s < kFaDv / 16; ++s) {
    const uint4 v = load16(a.dOb + qrow * kFaDv + 16 * s + 8 * hf);
    go[s] = *(const bf16x8*)&v;
  }
  const float2 sd = a.stat[qrow];
  const int i_last = min(qb * kFaTok + kFaTok - 1, T - 1);
  const int n_kt = i_last / kFaKeys + 1;
  const uint16_t* kbase = a.Kb + ((size_t)g * a.n_rows + sq.x) * kFaDqk;
  const uint16_t* vbase = a.Vb + ((size_t)g * a.n_rows + sq.x) * kFaDv;
  KvStage stage;
  f32x16 dQT[kFaDqk / 32];
#pragma unroll
  for (int mb = 0; mb < kFaDqk / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQT[mb][r] = 0.f;
  const int s16 = lane & 15, dblk = (lane >> 4) & 1;
  // Tile kt + 1 waits in registers while tile kt is computed, and tile
  // kt + 2 is on its way: two tiles of load latency hidden.
  KvStage sb;
  stage.load(kbase, vbase, 0, T, tid);
  stage.store(k_st[0], v_st[0], tid);
  if (1 < n_kt) stage.load(kbase, vbase, 1, T, tid);
  __syncthreads();
  auto tile = [&](int kt, int buf, KvStage& next, KvStage& after) {
    if (kt + 2 < n_kt) after.load(kbase, vbase, kt + 2, T, tid);
    const char* ks = k_st[buf];
    const char* vs = v_st[buf];
    f32x16 sacc, dpacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = 0.f;
      dpacc[r] = 0.f;
    }
    const char* krow = ks + n * kKPitch + 16 * hf;
#pragma unroll
    for (int s = 0; s < kQkSteps; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow + 32 * s), q[s], sacc,
                                                     0, 0, 0);
    const char* vrow = vs + n * kVPitch + 16 * hf;
#pragma unroll
    for (int s = 0; s < kFaDv / 16; ++s)
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vrow + 32 * s), go[s],
                                                      dpacc, 0, 0, 0);
    const int key0 = kt * kFaKeys + 4 * hf;
    const bool masked = kt * kFaKeys + kFaKeys - 1 > qb * kFaTok + 2 * wave;  // wave-uniform
    bf16x8 db[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + (r & 3);
      float p = __builtin_amdgcn_exp2f(sacc[r] - sd.x);
      if (masked && (key > i || key >= T)) p = 0.f;
      db[r >> 3][r & 7] = (__bf16)(p * (dpacc[r] - sd.y));
    }
    const char* tkb = ks + (4 * hf + (s16 >> 2)) * kKPitch + 32 * dblk + 8 * (s16 & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mb = 0; mb < kFaDqk / 32; ++mb) {
        const char* pa = tkb + 16 * kk * kKPitch + 64 * mb;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa + 8 * kKPitch));
        const bf16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dQT[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, db[kk], dQT[mb], 0, 0, 0);
      }
    if (kt + 1 < n_kt) next.store(k_st[buf ^ 1], v_st[buf ^ 1], tid);
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile(kt, 0, stage, sb);
    if (kt + 1 >= n_kt) break;
    tile(kt + 1, 1, sb, stage);
  }
  if (!valid) return;
  // dQ^ = tau sum dS K^ (the logits' scale of dS is the natural one)
  float* dq = a.dQh + qrow * kFaDqk + 4 * hf;
#pragma unroll
  for (int mb = 0; mb < kFaDqk / 32; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = dQT[mb][4 * r4 + c] * a.tau;
      *(f32x4*)(dq + 32 * mb + 8 * r4) = v;
    }
}

}  // namespace

bool train_mfma_shape(const Cfg& c) {
  return c.dtype == QKMLA_BF16 && c.hpg == kFaHpg && c.dc + c.dr == kFaDqk && c.dv == kFaDv;
}

hipError_t launch_flash_fwd(const Cfg& c, const FlashSeqs& q, const void* Qb, const void* Kb,
                            const void* Vb, float* o, float* lse, hipStream_t s) {
  FaArgs a{(const uint16_t*)Qb, (const uint16_t*)Kb, (const uint16_t*)Vb, o, lse, q.seqs,
           q.n_rows, c.H, c.G};
  hipLaunchKernelGGL(flash_fwd_kernel,
                     dim3((q.max_len + kFaTok - 1) / kFaTok * c.G, 1, q.n_seq), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace qkmla

namespace qkmla {

int flash_bwd_splits(int n_seq, int max_len, int G) {
  const int64_t blocks = (int64_t)(max_len + 4 * kFaKeys - 1) / (4 * kFaKeys) * G * n_seq;
  int sp = 1;
  while (sp < kFbMaxSplits && blocks * sp < kFbTargetWgs) sp *= 2;
  return sp;
}

hipError_t launch_flash_bwd(const Cfg& c, const FlashSeqs& q, const void* Qb, const void* Kb,
                            const void* Vb, const float* o, const float* lse, const float* d_o,
                            void* dOb, void* stat, float* dKh, float* dV, float* dQh,
                            float* part, hipStream_t s) {
  const int rows_h = q.n_rows * c.H;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((rows_h + 3) / 4), dim3(256), 0, s, rows_h, o, lse,
                     d_o, (uint16_t*)dOb, (float2*)stat);
  const int sp = flash_bwd_splits(q.n_seq, q.max_len, c.G);
  const size_t nk = (size_t)q.n_rows * c.G * kFaDqk, nv = (size_t)q.n_rows * c.G * kFaDv;
  float* dKp = sp > 1 ? part : dKh;
  float* dVp = sp > 1 ? part + sp * nk : dV;
  FbArgs a{(const uint16_t*)Qb, (const uint16_t*)Kb, (const uint16_t*)Vb, (const uint16_t*)dOb,
           (const float2*)stat, dKh, dV, dQh, q.seqs, q.n_rows, c.H, c.G, c.tau, dKp, dVp, sp};
  hipLaunchKernelGGL(flash_bwd_kv_kernel,
                     dim3((q.max_len + 4 * kFaKeys - 1) / (4 * kFaKeys) * c.G * sp, 1, q.n_seq),
                     dim3(256), 0, s, a);
  if (sp > 1) {
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((nk / 4 + 255) / 256)), dim3(256), 0, s,
                       nk / 4, sp, (const f32x4*)dKp, (f32x4*)dKh);
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((nv / 4 + 255) / 256)), dim3(256), 0, s,
                       nv / 4, sp, (const f32x4*)dVp, (f32x4*)dV);
  }
  hipLaunchKernelGGL(flash_bwd_q_kernel,
                     dim3((q.max_len + kFaTok - 1) / kFaTok * c.G, 1, q.n_seq), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace qkmla
