// Internal declarations shared by the host library and the HIP kernels.
// Everything here targets gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qkmla.h"

namespace qkmla {

// Normalised layer description used by every launcher.
struct Cfg {
  int H, G, r, dc, dr, dv;
  int dtype;     // QKMLA_F32 / QKMLA_BF16
  int qk_norm;
  float eps;
  float tau;     // softmax scale (already defaulted)
  float base;    // RoPE base
  int hpg;       // heads per group
};

// RoPE inverse frequencies theta_i = base^(-2i/d_r), i < d_r/2, in double.
// Formed once on the host per call and passed by value to the kernels that
// rotate, so no kernel evaluates a double-precision power.
constexpr int kMaxRopePairs = 128;
struct RopeFreq {
  double f[kMaxRopePairs];
};
RopeFreq rope_freq(int dr, float base);

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Token tile of the bf16 MFMA decode (rows staged in LDS per step).
constexpr int kTile = 32;
// Partial slots per decode workgroup (first and last sequence segment).
constexpr int kSlotsPerWg = 2;
// Bytes of one partial slot: the running max m and sum l of each head in
// fp32, the unnormalised O of each head in bf16 (it is rounded once, like the
// softmax weights, and the merge accumulates in fp32), head-major [H][r].
__host__ __device__ constexpr size_t kPartialSlotBytes(int H, int r) {
  return (size_t)H * 8 + (size_t)H * r * 2;
}

// Index of element (head h, dim d) of sequence b's bf16 query operands, q~
// (D = r) or the RoPE query (D = d_r), as the MFMA decode reads them: for each
// wavefront's 32 heads and each K-step of 16 dims, the 64 lanes' 16-byte B
// operands lie contiguous (lane n + 32 hf: head 32 j + n, dims 16 s + 8 hf ..
// + 8), so that one load instruction reads 1 KB in one piece.
__host__ __device__ __forceinline__ size_t qop_index(int b, int H, int D, int h, int d) {
  return ((((size_t)b * (H / 32) + h / 32) * (D / 16) + d / 16) * 64 + ((d >> 3) & 1) * 32 +
          (h & 31)) * 8 + (d & 7);
}

// ---- workspace layout of the bf16 MFMA decode ------------------------------
struct WsLayout {
  size_t q_tilde;    // bf16 operand order (qop_index, D = r); fp32 path: f32 [B][H][r]
  size_t alpha_q;    // f32  [B][H]   (tau*log2e folded in)
  size_t q_rope;     // bf16 operand order (qop_index, D = d_r); fp32 path: f32 [B][H][d_r]
                     // (normalised, rotated, tau*log2e folded in)
  size_t partials;   // [n_wg][kSlotsPerWg] slots of kPartialSlotBytes(H, r):
                     //   m[H] f32, l[H] f32, O[H][r] bf16
  size_t plan;       // i32  [B+1]  tile prefix of the split plan (written by the decode)
  size_t total;
};
WsLayout ws_layout(const Cfg& c, int batch, int n_wg);

// ---- cache addressing ---------------------------------------------------------
// The latent, RoPE and alpha caches are pools of num_pages pages of page_size
// rows.  Row t of cache b is row t % page_size of page
// bt[b * max_blocks + t / page_size].  A contiguous cache [B][L_cap] is the
// case bt == nullptr, page_size = L_cap, page b for cache b.  The capacity of
// one cache is max_blocks * page_size rows.
struct Paging {
  const int32_t* bt;  // device block table [B][max_blocks], or nullptr
  int max_blocks;
  int page_size;
  int num_pages;
  __host__ __device__ int capacity() const { return max_blocks * page_size; }
  // Page holding rows [blk * page_size, (blk + 1) * page_size) of cache b;
  // -1 if the block-table entry is outside [0, num_pages).
  __device__ int page_of(int b, int blk) const {
    if (!bt) return b;
    const int page = bt[(size_t)b * max_blocks + blk];
    return (page >= 0 && page < num_pages) ? page : -1;
  }
  // Physical row of row t of cache b, or -1 (bad block-table entry).
  __device__ int64_t phys_row(int b, int t) const {
    const int blk = t / page_size;
    const int page = page_of(b, blk);
    return page < 0 ? -1 : (int64_t)page * page_size + (t - blk * page_size);
  }
};
inline Paging contiguous_paging(int batch, int L_cap) { return Paging{nullptr, 1, L_cap, batch}; }

// ---- training / prefill (explicit form) ---------------------------------------
struct TrainPtrs {  // layer inputs (dtype = storage type unless noted)
  const void* c;       // [B][T][r]
  const void* q_c;     // [B][T][H][d_c]
  const void* q_rope;  // [B][T][H][d_r]
  const void* k_rope;  // [B][T][d_r]
  const float* w_uk;   // [G][r][d_c] fp32
  const void* w_uv;    // [G][r][d_v]
  const float *gamma_q, *gamma_k, *gamma_q_rope, *gamma_k_rope;  // fp32
};
struct TrainGrads {  // fp32 gradients, same shapes as the inputs
  float *d_c, *d_q_c, *d_q_rope, *d_k_rope, *d_w_uk, *d_w_uv;
  float *d_gamma_q, *d_gamma_k, *d_gamma_q_rope, *d_gamma_k_rope;
};
// Byte offsets of the fp32 training intermediates (d_qk = d_c + d_r):
//   Qh [BT][H][d_qk], Kh [BT][G][d_qk], V [BT][G][d_v], Kraw [BT][G][d_c],
//   aq, aqr [BT][H], ak [BT][G], akr [BT], RoPE (cos, sin) [T][d_r/2]
//   (the forward needs these: fwd_total)
//   dQh, dKh, dV, Dsum [BT][H], dK [BT][G][d_c], dKr [BT][d_r], gamma partials.
//   (bf16 layer with the MFMA attention also: Qb [BT][H][d_qk] scaled by
//   tau*log2(e), Kb [G][BT][d_qk], Vb [G][BT][d_v], all bf16)
// Packed sequences: n_seq sequences over n_rows token rows, each at most
// max_len long; cu (device, [n_seq+1]) holds their start rows and the total,
// or is nullptr for n_seq sequences of exactly max_len rows.
struct TrainSeqs {
  int n_rows, n_seq, max_len;
  const int32_t* cu;
};
// The flash kernels' view: validated (start, len) per sequence.
struct FlashSeqs {
  int n_rows, n_seq, max_len;
  const int2* seqs;
};
struct TrainWs {
  size_t seqs, rpos, rlen;  // (start, len) [n_seq] int2; per row: position, sequence length
  size_t Qh, Kh, V, Kraw, aq, aqr, ak, akr, rope_cs, Qb, Kb, Vb;
  size_t Wk16;  // MFMA path: W^UK in bf16 hi [G][r][d_c], then lo
  size_t fwd_total;
  size_t dQh, dKh, dV, Dsum, dK, dKr, gamma_partial;
  size_t dOb, stat;  // MFMA backward: d_o bf16 [BT][H][d_v], (lse*log2 e, D) [BT][H]
  size_t dKb, dVb;   // MFMA backward: dk, dV in bf16 [BT][G][d_c], [BT][G][d_v]
  size_t fb_part;    // MFMA backward, split key side: [S][BT][G][d_c + d_r], then [S][BT][G][d_v]
  size_t total;
};
TrainWs train_ws_layout(const Cfg& c, const TrainSeqs& q);
// The layer shape the MFMA attention is compiled for (bf16, 16 heads per
// group, d_c + d_r = 192, d_v = 128).
bool train_mfma_shape(const Cfg& c);
hipError_t launch_flash_fwd(const Cfg& c, const FlashSeqs& q, const void* Qb, const void* Kb,
                            const void* Vb, float* o, float* lse, hipStream_t s);
// dK^ and dV (key side) and dQ^ (query side) of the attention, fp32, in the
// row-major layouts of the row-parallel kernels.  The key side runs in
// S = flash_bwd_splits(...) token ranges; when S > 1 `part` holds their
// partial sums (S (d_c + d_r + d_v) floats per row and group), added in a
// fixed order.
int flash_bwd_splits(int n_seq, int max_len, int G);
hipError_t launch_flash_bwd(const Cfg& c, const FlashSeqs& q, const void* Qb, const void* Kb,
                            const void* Vb, const float* o, const float* lse, const float* d_o,
                            void* dOb, void* stat, float* dKh, float* dV, float* dQh,
                            float* part, hipStream_t s);

// ---- bf16 MFMA GEMM (training projections) --------------------------------------
// Operand element (mn, k) of batch z sits at p + z*batch_stride +
//   K-contiguous:  mn*ld + (k / kgrp)*kgrp_stride + k % kgrp  (kgrp a multiple of 8)
//   MN-contiguous: k*ld + mn                                  (ld, MN multiples of 8)
struct GemmOperand {
  const uint16_t* p;
  int64_t ld;
  int kgrp;
  int64_t kgrp_stride;
  int64_t batch_stride;
};
// C[z][m][n] = (C[z][m][n] if accumulate) + sum_k A[z][m][k] B[z][k][n], fp32 C at
// C + z*c_batch_stride + m*ldc + n.
struct GemmArgs {
  GemmOperand A, B;
  float* C;
  int64_t ldc, c_batch_stride;
  int M, N, K;
  int accumulate;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_kc, bool b_kc, int batch, hipStream_t s);

// ---- launchers (each enqueues on `stream`; returns the launch error) -------
hipError_t launch_absorb(const Cfg& c, const float* w_uk, const float* gq, const float* gk,
                         void* w_qabs, hipStream_t s);
hipError_t launch_append(const Cfg& c, int batch, int n_new, const void* c_new,
                         const void* k_rope_new, const float* w_uk, const float* gkr,
                         const int32_t* positions, const Paging& pg, void* lat, void* rope,
                         float* alpha, int32_t* status, hipStream_t s);
// Decode launchers take `batch` sequences with `s_q` query rows each: query
// row i of sequence b is virtual sequence b*s_q + i (its q rows, q~ rows and
// outputs), at position seq_lens[b] - s_q + i over cache b (see virt_len).
hipError_t launch_qprep(const Cfg& c, int batch, int s_q, const void* q_c, const void* q_rope,
                        const void* w_qabs, const float* gqr, const int32_t* seq_lens,
                        const Paging& pg, const WsLayout& ws, void* workspace, int32_t* status,
                        hipStream_t s);
hipError_t launch_decode_mfma(const Cfg& c, int batch, int s_q, const int32_t* seq_lens,
                              const Paging& pg, const void* lat, const void* rope,
                              const float* alpha, const WsLayout& ws, void* workspace, int n_wg,
                              float* o_lat, float* lse, hipStream_t s);
// Launch k on stream s and return the launch's status.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, A... a) {
  k<<<grid, block, 0, s>>>(static_cast<P>(a)...);
  return hipGetLastError();
}

// Whether launch_out_proj takes the MFMA kernel, which reads o_lat and W^UV
// as 16-byte vectors (so both must be 16-byte aligned).
bool out_proj_uses_mfma(const Cfg& c);
hipError_t launch_merge(const Cfg& c, int batch, int s_q, const WsLayout& ws, void* workspace,
                        int n_wg, float* o_lat, float* lse, hipStream_t s);
hipError_t launch_decode_generic(const Cfg& c, int batch, int s_q, const int32_t* seq_lens,
                                 const Paging& pg, const void* lat, const void* rope,
                                 const float* alpha, const WsLayout& ws, void* workspace,
                                 float* o_lat, float* lse, hipStream_t s);
hipError_t launch_train_forward(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                                const TrainWs& ws, void* workspace, float* o, float* lse,
                                int32_t* status, hipStream_t s);
hipError_t launch_train_backward(const Cfg& c, const TrainSeqs& q, const TrainPtrs& in,
                                 const float* o, const float* lse, const float* d_o,
                                 const TrainWs& ws, void* workspace, const TrainGrads& gr,
                                 int32_t* status, hipStream_t s);
hipError_t launch_out_proj(const Cfg& c, int batch, const float* o_lat, const void* w_uv,
                           float* out, hipStream_t s);

}  // namespace qkmla
