// Device-side split plan of the bf16 decode.
//
// Work is measured in token tiles.  Sequence b holds n_b = ceil(L_b / kTile)
// tiles (0 if L_b is outside [1, L_cap]); the tiles of all sequences are laid
// end to end and workgroup p of n_wg takes tiles [floor(p N / n_wg),
// floor((p+1) N / n_wg)), N = sum n_b.  A workgroup's range may cross
// sequence boundaries; each piece of one sequence is a segment.  A segment
// that covers its whole sequence writes the final output directly.  Otherwise
// it writes a partial (m, l, O) into slot 0 if it is the first segment of its
// workgroup and slot 1 if it is a later one (only the last can be partial),
// and the merge kernel combines the partials of the sequence.
#pragma once

#include "qkmla_internal.h"

namespace qkmla {

constexpr int kMaxBatch = 4096;

__host__ __device__ __forceinline__ int tiles_of(int L, int L_cap) {
  return (L >= 1 && L <= L_cap) ? (L + kTile - 1) / kTile : 0;
}

// Length of virtual sequence v when every sequence carries s_q query rows:
// row i = v % s_q of sequence b = v / s_q is the token at position
// L_b - s_q + i and attends cache rows 0..L_b - s_q + i (causal).  With
// s_q = 1 this is seq_lens[v].  A sequence length outside [1, L_cap] makes all
// of its rows invalid (length 0).
__host__ __device__ __forceinline__ int virt_len(const int32_t* seq_lens, int v, int s_q, int L_cap) {
  const int L = seq_lens[v / s_q];
  if (L < 1 || L > L_cap) return 0;
  return L - s_q + 1 + v % s_q;
}

// Exclusive prefix over tiles_of(virt_len(v)) into P[0..B] (LDS), block-wide,
// for the B virtual sequences.  Must be called by every thread of the block
// (64, 128 or 256 threads).
__device__ void build_tile_prefix(const int32_t* __restrict__ seq_lens, int B, int s_q, int L_cap,
                                  int* P) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per = (B + nthr - 1) / nthr;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < B) local += tiles_of(virt_len(seq_lens, b, s_q, L_cap), L_cap);
  }
  // inclusive scan of `local` across the block
  int lane = tid & 63, wave = tid >> 6;
  int v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int excl = before + v - local;
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < B) {
      P[b] = excl;
      excl += tiles_of(virt_len(seq_lens, b, s_q, L_cap), L_cap);
    }
  }
  if (tid == nthr - 1) P[B] = before + v;
  __syncthreads();
}

__host__ __device__ __forceinline__ int64_t wg_start(int p, int64_t N, int n_wg) {
  return ((int64_t)p * N) / n_wg;
}

// Workgroup whose range holds tile x (0 <= x < N).
__host__ __device__ __forceinline__ int wg_of(int64_t x, int64_t N, int n_wg) {
  return (int)(((x + 1) * n_wg - 1) / N);
}

// Largest b with P[b] <= x (the sequence holding tile x); P has B+1 entries.
__host__ __device__ __forceinline__ int seq_of(const int* P, int B, int64_t x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (P[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Partial slot written for sequence b by workgroup p (p_lo <= p <= p_hi of b),
// or -1 if p holds no tile of b (an empty range between p_lo and p_hi).
// Mirrors the decode kernel: a workgroup's first segment uses slot 0, a later
// one slot 1.
__host__ __device__ __forceinline__ int merge_slot_of(int64_t Pb, int p_lo, int64_t N, int n_wg,
                                                      int p) {
  if (p == p_lo) return wg_start(p_lo, N, n_wg) == Pb ? 0 : 1;
  return wg_start(p, N, n_wg) == wg_start(p + 1, N, n_wg) ? -1 : 0;
}
__host__ __device__ __forceinline__ int merge_slot(const int* P, int b, int64_t N, int n_wg,
                                                   int p) {
  return merge_slot_of(P[b], wg_of(P[b], N, n_wg), N, n_wg, p);
}

}  // namespace qkmla
