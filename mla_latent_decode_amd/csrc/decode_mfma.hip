// Split-KV flash-decoding of QK-Normed MLA over the bf16 latent / RoPE caches
// and the fp32 alpha cache, on gfx950 MFMA.
//
// What one workgroup computes, per token t of its range and head h
// (g = g(h); "QK-Normed MLA: QK normalization without full key caching",
// technical summary, Methodology: decode-logit formula and row-column scaling,
// Blockwise Normalization):
//   S_c[t,h] = q~_h . c_t                (K = r = 512, MFMA)
//   S_r[t,h] = q^R_h . k^R_t             (K = d_r = 64, MFMA)
//   l[t,h]   = S_c * (alpha^q_h * alpha^k_{t,g}) + S_r       (exp2 domain)
//   online softmax over t, O[h,:] += sum_t p[t,h] c_t        (K = 32 tokens, MFMA)
// Plain MLA (QKN = false) uses one K = r + d_r accumulator, no alpha.
//
// Shape: r = 512, d_r = 64, 32 heads per wavefront, NW = H/32 wavefronts per
// workgroup (all heads of a token are handled by one workgroup, so every
// cache byte is read from HBM once).  Token tiles of 32 rows are staged in LDS
// by direct global->LDS loads (3 stages).  MFMA 32x32x16 bf16 layouts
// (gfx950): A lane l holds A[m=l%32][k=8(l/32)+j]; B lane l holds
// B[k=8(l/32)+j][n=l%32]; D lane l reg i holds D[8(i/4)+4(l/32)+i%4][l%32].
//   QK:  S^T (tokens x heads) = C (tokens x 512) . Q~^T ; A from LDS rows,
//        B = q~ kept in registers for the whole segment.
//   PV:  O^T (dims x heads) += C^T (dims x tokens) . P^T ; B = P taken
//        straight from the S^T accumulator (token order permuted to match),
//        A = C^T read with ds_read_b64_tr_b16: within each 16-lane group,
//        lane i receives element i%4 of the 8-byte loads of lanes 4e + i/4
//        (e = 0..3), which turns 4 token rows into 4 tokens of one dim.
#include "device_common.h"
#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {

namespace {

constexpr int kR = 512;
constexpr int kDr = 64;
constexpr int kStages = 3;
constexpr int kLatRow = kR * 2 + 48;          // 1072 B: 1 KB row + 48 B pad
constexpr int kLatBytes = kTile * kLatRow;    // 33.5 KB
constexpr int kRopeBytes = kTile * kDr * 2;   // 4 KB
constexpr int kAlphaMaxG = 8;
constexpr int kAlphaBytes = kTile * kAlphaMaxG * 4;  // 1 KB
constexpr int kStageBytes = kLatBytes + kRopeBytes + kAlphaBytes;
// p = 2^(logit - m_ref) may exceed 1; a segment is streamed again with a
// raised reference only if some p would exceed 2^kOverflowLog2.
constexpr float kOverflowLog2 = 64.0f;


// Wait until at most N vector memory operations of this wavefront are in
// flight.  s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[5:4] << 14; expcnt and lgkmcnt are left at "no wait".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that drains this wave's LDS operations (lgkmcnt(0)) but
// leaves its global->LDS prefetches in flight (vmcnt untouched, unlike
// __syncthreads).
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt=63, expcnt=7, lgkmcnt=0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Args {
  const int32_t* seq_lens;
  int B, H, G, L_cap, n_wg;
  const uint16_t* lat;
  const uint16_t* rope;
  const float* alpha;
  const uint16_t* q_tilde;
  const float* alpha_q;
  const uint16_t* q_rope;
  float* part;
  float* o_lat;
  float* lse;
};

// Loads per wavefront per tile (all wavefronts issue the same count).
template <bool QKN, int NW>
struct TileLoads {
  static constexpr int lat = kTile / NW;              // one 1 KB row per instruction
  static constexpr int rope = 4 / NW > 0 ? 4 / NW : 1;  // 8 rows per instruction
  static constexpr int alpha = QKN ? (4 / NW > 0 ? 4 / NW : 1) : 0;
  static constexpr int total = lat + rope + alpha;
};

// Issue the direct global->LDS loads of one tile into a stage buffer.
// LDS layout of a stage:
//   latent: token-major rows of kLatRow bytes (1 KB of data + 48 B pad); one
//           load instruction moves one row.  The 1072-byte stride (67 16-byte
//           units, 3 mod 16) spreads both the QK row reads and the transposed
//           PV reads over distinct bank groups.
//   rope:   chunk-major, position 32*c + t for 16-byte chunk c of token t.
//   alpha:  [g][32 tokens] floats.
template <bool QKN, int NW>
__device__ __forceinline__ void issue_tile(const Args& a, char* stage, const uint16_t* lat_b,
                                           const uint16_t* rope_b, const float* alpha_b, int t0,
                                           int L, int wave, int lane) {
  // Scalar row base + zero-extended 32-bit lane offset lets the compiler use
  // the SGPR-base form of the load.
  const uint32_t lane16 = (uint32_t)lane << 4;
#pragma unroll
  for (int i = 0; i < TileLoads<QKN, NW>::lat; ++i) {
    const int tr = wave + i * NW;
    const int row = min(t0 + tr, L - 1);
    const char* rowp = (const char*)lat_b + (size_t)row * (kR * 2);
    __builtin_amdgcn_global_load_lds(QK_GLB(void, rowp + lane16),
                                     QK_LDS(void, stage + tr * kLatRow), 16, 0, 0);
  }
  const int t = lane & 31;
  const uint32_t rrow = (uint32_t)min(t0 + t, L - 1);
  const uint32_t rope_off = rrow * (kDr * 2) + ((uint32_t)(lane >> 5) << 4);
#pragma unroll
  for (int i = 0; i < TileLoads<QKN, NW>::rope; ++i) {
    const int blk = wave + i * NW;  // chunks 2*blk, 2*blk+1
    __builtin_amdgcn_global_load_lds(QK_GLB(void, (const char*)rope_b + blk * 32 + rope_off),
                                     QK_LDS(void, stage + kLatBytes + blk * 1024), 16, 0, 0);
  }
  if (QKN) {
    const uint32_t a_off = rrow * (uint32_t)(a.G * 4);
#pragma unroll
    for (int i = 0; i < TileLoads<QKN, NW>::alpha; ++i) {
      const int blk = wave + i * NW;  // groups 2*blk, 2*blk+1
      int g = 2 * blk + (lane >> 5);
      g = g < a.G ? g : a.G - 1;
      __builtin_amdgcn_global_load_lds(QK_GLB(void, (const char*)alpha_b + a_off + (uint32_t)(g * 4)),
                                       QK_LDS(void, stage + kLatBytes + kRopeBytes + blk * 256),
                                       4, 0, 0);
    }
  }
}

template <bool QKN, int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ int P[kMaxBatch + 1];
  __shared__ int restart_flag;
  volatile int* restart = &restart_flag;
  if (threadIdx.x == 0) restart_flag = 0;
  build_tile_prefix(a.seq_lens, a.B, a.L_cap, P);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5;        // which half of the 64 lanes
  const int n = lane & 31;         // head column within the wave
  const int head = wave * 32 + n;  // head index in the layer
  const int g = (head * a.G) / a.H;
  const int64_t N = __builtin_amdgcn_readfirstlane(P[a.B]);
  const int p = blockIdx.x;
  int64_t x = wg_start(p, N, a.n_wg);
  const int64_t e = wg_start(p + 1, N, a.n_wg);
  bool first_seg = true;

  while (x < e) {
    const int b = __builtin_amdgcn_readfirstlane(seq_of(P, a.B, x));
    const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    const int64_t s0 = __builtin_amdgcn_readfirstlane(P[b]);
    const int64_t s1 = __builtin_amdgcn_readfirstlane(P[b + 1]);
    const int64_t seg_end = e < s1 ? e : s1;
    const int tile_first = (int)(x - s0);
    const int nt = (int)(seg_end - x);

    // Query operands for this sequence, kept in registers for the segment.
    const size_t qrow = (size_t)b * a.H + head;
    bf16x8 qt[kR / 16];
#pragma unroll
    for (int s = 0; s < kR / 16; ++s)
      qt[s] = *(const bf16x8*)(a.q_tilde + qrow * kR + s * 16 + hf * 8);
    bf16x8 qr[kDr / 16];
#pragma unroll
    for (int s = 0; s < kDr / 16; ++s)
      qr[s] = *(const bf16x8*)(a.q_rope + qrow * kDr + s * 16 + hf * 8);
    const float aq = QKN ? a.alpha_q[qrow] : 1.0f;
    const size_t seq_row0 = (size_t)b * a.L_cap;
    const uint16_t* lat_b = a.lat + seq_row0 * kR;
    const uint16_t* rope_b = a.rope + seq_row0 * kDr;
    const float* alpha_b = QKN ? a.alpha + seq_row0 * a.G : nullptr;

    f32x16 O[kR / 32];
    float m_ref = -INFINITY, l_run = 0.f;
    bool have_ref = false;
    for (;;) {  // one pass over the segment; repeated only if a logit overflows the reference
#pragma unroll
      for (int ii = 0; ii < kR / 32; ++ii)
#pragma unroll
        for (int j = 0; j < 16; ++j) O[ii][j] = 0.f;
      l_run = 0.f;
#pragma unroll
      for (int j = 0; j < kStages - 1; ++j)
        if (j < nt) issue_tile<QKN, NW>(a, smem + j * kStageBytes, lat_b, rope_b, alpha_b,
                                        (tile_first + j) * kTile, L, wave, lane);
      int cur = 0;
      for (int i = 0; i < nt; ++i) {
        if (i + 1 < nt) wait_vmcnt<TileLoads<QKN, NW>::total>();
        else wait_vmcnt<0>();
        block_sync();
        const int nxt = cur == 0 ? kStages - 1 : cur - 1;
        if (i + kStages - 1 < nt)
          issue_tile<QKN, NW>(a, smem + nxt * kStageBytes, lat_b, rope_b, alpha_b,
                              (tile_first + i + kStages - 1) * kTile, L, wave, lane);
        const char* st = smem + cur * kStageBytes;
        cur = cur == kStages - 1 ? 0 : cur + 1;
        const int t0 = (tile_first + i) * kTile;
        // ---- logits S^T[32 tokens][32 heads] ----
        f32x16 sc, sr;
#pragma unroll
        for (int j = 0; j < 16; ++j) { sc[j] = 0.f; sr[j] = 0.f; }
        {
          const int m = lane & 31;
          const char* row = st + m * kLatRow + hf * 16;
#pragma unroll
          for (int s = 0; s < kR / 16; ++s) {
            bf16x8 av = *(const bf16x8*)(row + s * 32);
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qt[s], sc, 0, 0, 0);
          }
          const char* rrow = st + kLatBytes + (32 * hf + m) * 16;
#pragma unroll
          for (int s = 0; s < kDr / 16; ++s) {
            bf16x8 av = *(const bf16x8*)(rrow + s * 1024);
            if (QKN) sr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qr[s], sr, 0, 0, 0);
            else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qr[s], sc, 0, 0, 0);
          }
        }

        // ---- row-column scaling, mask, softmax weights (exp2 domain) ----
        float lg[16];
        if (QKN) {
          const float* al = (const float*)(st + kLatBytes + kRopeBytes) + g * 32 + 4 * hf;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 ak = *(const f32x4*)(al + 8 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) lg[4 * q + j] = sc[4 * q + j] * (aq * ak[j]) + sr[4 * q + j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) lg[j] = sc[j];
        }
        const int valid = L - t0;  // tokens < valid are real
        if (valid < kTile) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int tok = 8 * (j >> 2) + 4 * hf + (j & 3);
            if (tok >= valid) lg[j] = -INFINITY;
          }
        }
        float mt = lg[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mt = fmaxf(mt, lg[j]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        if (!have_ref) {  // first tile of the segment sets the per-head reference
          m_ref = mt;
          have_ref = true;
        }
        if (__ballot(mt > m_ref + kOverflowLog2) != 0) {
          m_ref = fmaxf(m_ref, mt);
          *restart = 1;
        }
        bf16x8 pb[2];
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const __bf16 v = (__bf16)exp2f(lg[j] - m_ref);
          pb[j >> 3][j & 7] = v;
          ls += (float)v;
        }
        l_run += ls;

        // ---- O^T[512 dims][32 heads] += C^T . P^T ----
        {
          // lane (in its 16-lane group): token 4*hf + (s16>>2) of the 16-token
          // step, 4 dims at 32*mb + 16*dblk + 4*(s16&3)
          const int s16 = lane & 15, dblk = (lane >> 4) & 1;
          const char* pvb = st + (4 * hf + (s16 >> 2)) * kLatRow + 32 * dblk + 8 * (s16 & 3);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int mb = 0; mb < kR / 32; ++mb) {
              const char* pa = pvb + (16 * ks) * kLatRow + 64 * mb;
              bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa));
              bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pa + 8 * kLatRow));
              bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], O[mb], 0, 0, 0);
            }
          }
        }
      }
      block_sync();
      if (!*restart) break;
      // A logit exceeded the reference by more than 2^kOverflowLog2: stream the
      // segment again with the raised reference (exact; never taken for
      // normalised logits).
      block_sync();
      if (threadIdx.x == 0) *restart = 0;
    }
    // ---- segment epilogue ----
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float m_run = m_ref;
    const bool complete = (x == s0) && (seg_end == s1);
    if (complete) {
      const float inv = 1.0f / l_tot;
      float* out = a.o_lat + qrow * kR;
#pragma unroll
      for (int mb = 0; mb < kR / 32; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v = {O[mb][4 * q] * inv, O[mb][4 * q + 1] * inv, O[mb][4 * q + 2] * inv,
                     O[mb][4 * q + 3] * inv};
          *(f32x4*)(out + 32 * mb + 8 * q + 4 * hf) = v;
        }
      if (hf == 0 && a.lse) a.lse[qrow] = (m_run + log2f(l_tot)) * kLn2;
    } else {
      const int slot = first_seg ? 0 : 1;
      float* sp = a.part + ((size_t)p * kSlotsPerWg + slot) * (size_t)a.H * (kR + 2);
      if (hf == 0) {
        sp[head] = m_run;
        sp[a.H + head] = l_tot;
      }
      float* Op = sp + 2 * a.H + (size_t)head * kR;
#pragma unroll
      for (int mb = 0; mb < kR / 32; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v = {O[mb][4 * q], O[mb][4 * q + 1], O[mb][4 * q + 2], O[mb][4 * q + 3]};
          *(f32x4*)(Op + 32 * mb + 8 * q + 4 * hf) = v;
        }
    }
    first_seg = false;
    x = seg_end;
    block_sync();  // all waves done with the stage buffers before the next segment
  }
}

}  // namespace

hipError_t launch_decode_mfma(const Cfg& c, int batch, const int32_t* seq_lens, int L_cap,
                              const void* lat, const void* rope, const float* alpha,
                              const WsLayout& ws, void* workspace, int n_wg, float* o_lat,
                              float* lse, hipStream_t s) {
  char* wsb = (char*)workspace;
  Args a;
  a.seq_lens = seq_lens;
  a.B = batch;
  a.H = c.H;
  a.G = c.G;
  a.L_cap = L_cap;
  a.n_wg = n_wg;
  a.lat = (const uint16_t*)lat;
  a.rope = (const uint16_t*)rope;
  a.alpha = alpha;
  a.q_tilde = (const uint16_t*)(wsb + ws.q_tilde);
  a.alpha_q = (const float*)(wsb + ws.alpha_q);
  a.q_rope = (const uint16_t*)(wsb + ws.q_rope);
  a.part = (float*)(wsb + ws.partials);
  a.o_lat = o_lat;
  a.lse = lse;
  const int nw = c.H / 32;
  dim3 grid(n_wg), block(nw * 64);
  if (c.qk_norm) {
    if (nw == 4) decode_mfma_kernel<true, 4><<<grid, block, 0, s>>>(a);
    else if (nw == 2) decode_mfma_kernel<true, 2><<<grid, block, 0, s>>>(a);
    else return hipErrorInvalidValue;  // one-wavefront variant switched off
  } else {
    if (nw == 4) decode_mfma_kernel<false, 4><<<grid, block, 0, s>>>(a);
    else if (nw == 2) decode_mfma_kernel<false, 2><<<grid, block, 0, s>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qkmla
