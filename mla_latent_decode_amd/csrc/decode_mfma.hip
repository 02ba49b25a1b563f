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
// alpha^q_h (with the softmax scale and log2(e)) is already folded into q~ by
// the query preparation, so the row-column scaling is one FMA per logit.
//   softmax weights over t, O[h,:] += sum_t p[t,h] c_t       (K = 32 tokens, MFMA)
// Plain MLA (QKN = false) runs the same two sums and adds them, with no alpha.
//
// Shape: r = 512, d_r = 64, 32 heads per wavefront, NW = H/32 wavefronts per
// workgroup (all heads of a token are handled by one workgroup, so every
// cache byte is read from HBM once).  Token tiles of 32 rows are staged in LDS
// by direct global->LDS loads, three stages deep: while a tile is consumed the
// next two are in flight.  MFMA 32x32x16 bf16 layouts (gfx950): A lane l holds
// A[m=l%32][k=8(l/32)+j]; B lane l holds B[k=8(l/32)+j][n=l%32]; D lane l reg i
// holds D[8(i/4)+4(l/32)+i%4][l%32].
//   QK:  S^T (tokens x heads) = C (tokens x 512) . Q~^T ; A from LDS rows,
//        B = q~ kept in registers for the whole segment.
//   PV:  O^T (dims x heads) += C^T (dims x tokens) . P^T ; B = P taken
//        straight from the S^T accumulator (token order permuted to match),
//        A = C^T read with ds_read_b64_tr_b16: within each 16-lane group,
//        lane i receives element i%4 of the 8-byte loads of lanes 4e + i/4
//        (e = 0..3), which turns 4 token rows into 4 tokens of one dim.
//
// Register budget per lane (one wavefront per SIMD): the O^T accumulator
// (512 dims x 32 heads fp32) fills the 256 AGPRs and q~ takes 128 VGPRs; the
// RoPE query sits in LDS.  MFMA results always land in AGPRs here, so each
// step moves one O^T block (16 AGPRs) out to VGPRs and back while the logits
// occupy its registers.  The tile loop does not spill; the segment prologue
// and epilogue do, a few registers once per segment.
#include <type_traits>

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
// Epilogue transpose: a wave's 32 head rows of 512 bytes per round (128 fp32
// or 256 bf16 dims) plus 16 bytes of pad against bank conflicts; two such
// regions per stage buffer.
constexpr int kEpiRow = 512 + 16;
constexpr int kEpiRegion = 32 * kEpiRow;
constexpr int kEpiBatch = 8;  // LDS rows read ahead of their stores
static_assert(2 * kEpiRegion <= kStageBytes, "two epilogue regions per stage buffer");
// p = 2^(logit - m_ref) may exceed 1; a segment is streamed again with a
// raised reference only if some p would exceed 2^kOverflowLog2.
constexpr float kOverflowLog2 = 64.0f;

// The stage buffers are three separate LDS objects, each addressed through a
// compile-time stage index.  The compiler's wait-count insertion can then tell
// a direct global->LDS load into one stage from an LDS read of another, and
// the reads of the tile being consumed do not wait for the tiles in flight.
__shared__ __attribute__((aligned(1024))) char lds_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) char lds_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) char lds_stage2[kStageBytes];

// Set by a wave whose logits overflow the segment's reference, one word per
// wave so that no two waves write the same word; read by all after a barrier
// (every access is ordered by the barriers' memory clobbers).
__shared__ int lds_restart[4];

// The RoPE query of every head, as the B operands of the four RoPE K-steps:
// 16 bytes per lane, [wave][step][lane].  Kept in LDS rather than in VGPRs,
// which the q~ operands and the tile step fill.
constexpr int kQropeBytes = 4 * (kDr / 16) * 64 * 16;  // up to 4 wavefronts: 16 KB
__shared__ __attribute__((aligned(16))) char lds_qrope[kQropeBytes];

template <int S>
__device__ __forceinline__ char* stage_buf() {
  static_assert(S >= 0 && S < kStages, "stage index");
  if constexpr (S == 0) return lds_stage0;
  else if constexpr (S == 1) return lds_stage1;
  else return lds_stage2;
}

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

// Workgroup index in the plan for hardware workgroup `hw` of `n`.  Workgroups
// are dispatched round-robin over the 8 XCDs, each with its own L2; this
// numbering gives every XCD a contiguous block of plan ranges, so the
// workgroups of one sequence share the L2 that holds its queries.
__device__ __forceinline__ int plan_wg(int hw, int n) {
  constexpr int kXcds = 8;
  if (n % kXcds != 0) return hw;
  return (hw % kXcds) * (n / kXcds) + hw / kXcds;
}

struct Args {
  const int32_t* seq_lens;
  int B;    // virtual sequences: batch * s_q (one per query row)
  int s_q;  // query rows per sequence
  int H, G, n_wg;
  Paging pg;  // where cache rows live (pages of a multiple of kTile rows, or contiguous)
  const uint16_t* lat;
  const uint16_t* rope;
  const float* alpha;
  const uint16_t* q_tilde;
  const uint16_t* q_rope;
  char* part;   // partial slots, kPartialSlotBytes(H, r) each
  int32_t* plan;  // [B+1] tile prefix, for the merge
  float* o_lat;
  float* lse;
};

// Row m of a tile's logits (the QK accumulator's token index) is token
// slot_token(m) of the tile: bits (m4 m3 m2 m1 m0) -> (m4 m1 m0 m3 m2).  The
// RoPE and alpha parts of a stage are stored in this slot order; latent rows
// are stored in token order and the QK reads pick row slot_token(m).  With
// the 1072-byte row stride (268 dwords, 12 mod 64 banks) this keeps both
// latent read patterns free of LDS bank conflicts:
//   QK (ds_read_b128, 16 lanes a pass): lanes m = 0..15 read rows
//     slot_token(m), 16 distinct values mod 16, so 16 distinct 4-bank groups;
//   PV (ds_read_b64_tr_b16, 32 lanes a pass): the four token rows that one
//     16-lane group transposes are accumulator rows 4e + c0 (e = 0..3), i.e.
//     latent rows 4e' + c1, 48 banks apart mod 64: four disjoint 16-bank runs.
__host__ __device__ constexpr int slot_token(int m) {
  return (m & 16) | ((m & 3) << 2) | ((m >> 2) & 3);
}
constexpr bool slot_token_is_a_permutation() {
  unsigned seen = 0;
  for (int m = 0; m < kTile; ++m) seen |= 1u << slot_token(m);
  return kTile == 32 && seen == 0xffffffffu;
}
static_assert(slot_token_is_a_permutation(), "slot order covers the 32 tokens of a tile");

// Loads per wavefront per tile (all wavefronts issue the same count).
template <bool QKN, int NW>
struct TileLoads {
  static constexpr int lat = kTile / NW;              // one 1 KB row per instruction
  static constexpr int rope = 4 / NW > 0 ? 4 / NW : 1;  // 8 rows per instruction
  static constexpr int alpha = QKN ? (4 / NW > 0 ? 4 / NW : 1) : 0;
  static constexpr int total = lat + rope + alpha;
};

// The sequence a segment belongs to (wave-uniform values).
struct Seq {
  const char* lat;    // latent row pool, 1 KB per row
  const char* rope;   // RoPE row pool, 128 B per row
  const char* alpha;  // alpha row pool, 4*G B per row
  int cb;             // cache (sequence of the batch) whose rows are read
  int last_tile;      // index of the sequence's last tile (from the tile prefix)
  int L;              // length of the (virtual) sequence; read only for its last tile
};

// Per-wavefront state carried across the tiles of a segment.
struct Wave {
  bf16x8 qt[kR / 16];   // q~ of the wave's 32 heads (B operand, K = latent dims)
  f32x16 O[kR / 32];    // O^T accumulator: 16 blocks of 32 dims x 32 heads
  float m_ref;          // reference max of the lane's head (exp2 domain)
  float l_run;          // running sum of the softmax weights (this lane's tokens)
  bool have_ref;
};

// Buffer descriptor (raw: stride 0) for `bytes` bytes from `base`.  Dword 3
// sets the 32-bit data format that untyped gfx9 buffer loads require.  The
// tile loads go through buffer instructions rather than global ones: the
// compiler counts a global load into LDS as a possible LDS access of unknown
// order, and while one is in flight it turns every LDS wait into a full drain,
// which would stall the MFMA pipelines on each wait.
constexpr int kBufDword3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufDword3);
}

// Issue the direct global->LDS loads of tile `tile` (of its sequence) into
// stage S.  LDS layout of a stage:
//   latent: token-major rows of kLatRow bytes (1 KB of data + 48 B pad); one
//           load instruction moves one row.
//   rope:   chunk-major, position 32*c + m for 16-byte chunk c of the token
//           in slot m (token slot_token(m)).
//   alpha:  [g][32 slots] floats, slot m holding token slot_token(m).
// Rows past the end of the sequence repeat its last row (masked later).
template <bool QKN, int NW, int S>
__device__ __forceinline__ void issue_tile(const Seq& sq, const Paging& pg, int G, int tile,
                                           int wave, int lane) {
  char* st = stage_buf<S>();
  // Opaque copies of the tile's first row and the lane offset keep the address
  // arithmetic here, as a scalar row base plus a 32-bit lane offset (the
  // scalar-base form of the load).  Otherwise the first two tiles' per-lane
  // 64-bit addresses are hoisted out of the segment's re-stream loop and stay
  // live, in spilled registers, across the whole segment.
  int t0 = tile * kTile;
  asm volatile("" : "+s"(t0));
  uint32_t lane16 = (uint32_t)lane << 4;
  asm volatile("" : "+v"(lane16));
  // The tile lies in one page (page sizes are multiples of kTile; a contiguous
  // cache is one page per sequence).  A block-table entry outside the pool
  // reads page 0 instead; q-prep has reported it.
  int64_t prow0 = (int64_t)sq.cb * pg.page_size + t0;  // contiguous: page cb, no table
  if (pg.bt) {
    const int blk = t0 / pg.page_size;
    // Table entry through the constant address space: a scalar load, waited
    // on by lgkmcnt rather than vmcnt, so the tile loads in flight keep going.
    const __attribute__((address_space(4))) int32_t* row =
        (const __attribute__((address_space(4))) int32_t*)(pg.bt + (size_t)sq.cb * pg.max_blocks);
    int page = row[blk];
    page = (page >= 0 && page < pg.num_pages) ? page : 0;
    prow0 = (int64_t)page * pg.page_size + (t0 - blk * pg.page_size);
  }
  // Rows past the sequence repeat its last row; only its last tile has such
  // rows, and only there is the length needed (a uniform branch, so the
  // length's load is waited for only on that tile).
  int last = kTile;
  if (tile == sq.last_tile) {
    asm volatile("" ::: "memory");
    last = sq.L - 1 - t0;
  }
  // One buffer descriptor per part of the tile, based at the tile's first row
  // and sized to the tile; the row and lane offsets go in the scalar and
  // vector offset fields.
  const __amdgpu_buffer_rsrc_t lat_rsrc =
      tile_rsrc(sq.lat + prow0 * (kR * 2), kTile * kR * 2);
#pragma unroll
  for (int i = 0; i < TileLoads<QKN, NW>::lat; ++i) {
    const int tr = wave + i * NW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lat_rsrc, QK_LDS(void, st + tr * kLatRow), 16,
                                             (int)lane16, min(tr, last) * (kR * 2), 0, 0);
  }
  int slot = lane & 31;
  asm volatile("" : "+v"(slot));  // recomputed per tile rather than held live
  const uint32_t rr = (uint32_t)min(slot_token(slot), last);
  const __amdgpu_buffer_rsrc_t rope_rsrc =
      tile_rsrc(sq.rope + prow0 * (kDr * 2), kTile * kDr * 2);
  const uint32_t rope_off = rr * (kDr * 2) + ((uint32_t)(lane >> 5) << 4);
#pragma unroll
  for (int i = 0; i < TileLoads<QKN, NW>::rope; ++i) {
    const int blk2 = wave + i * NW;  // chunks 2*blk2, 2*blk2+1
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rope_rsrc, QK_LDS(void, st + kLatBytes + blk2 * 1024),
                                             16, (int)rope_off, blk2 * 32, 0, 0);
  }
  if constexpr (QKN) {
    const __amdgpu_buffer_rsrc_t alpha_rsrc =
        tile_rsrc(sq.alpha + prow0 * (G * 4), kTile * G * 4);
    const uint32_t a_off = rr * (uint32_t)(G * 4);
#pragma unroll
    for (int i = 0; i < TileLoads<QKN, NW>::alpha; ++i) {
      const int blk2 = wave + i * NW;  // groups 2*blk2, 2*blk2+1
      int g = 2 * blk2 + (lane >> 5);
      g = g < G ? g : G - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          alpha_rsrc, QK_LDS(void, st + kLatBytes + kRopeBytes + blk2 * 256), 4,
          (int)(a_off + (uint32_t)(g * 4)), 0, 0, 0);
    }
  }
}

// The two halves of a head (lanes l and l ^ 32) combined: v_permlane32_swap
// trades lanes 32..63 of one register with lanes 0..31 of another, so with x
// in both, the two results hold x of this lane and of its partner in some
// order in every lane; their sum or max is the same in both lanes.  No LDS
// and no lane index are needed.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// This lane's index in its wavefront, computed where it is used: an opaque
// computation that the compiler cannot share with an earlier one, which it
// would otherwise keep live (in a spilled register) across the tile loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Order fence: the compiler's scheduler keeps instructions on their side, so
// the software pipelines below issue in the order they are written.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

constexpr int kRopeSteps = kDr / 16;            // 4 K-steps over the RoPE dims
constexpr int kQkSteps = kR / 16 + kRopeSteps;  // 36 K-steps of 16 (RoPE, then latent)
constexpr int kQkAhead = 4;                     // LDS reads in flight ahead of the QK MFMAs
constexpr int kPvSteps = 2 * (kR / 32);         // 32: 2 token halves x 16 dim blocks
constexpr int kPvAhead = 3;                     // C^T operands in flight ahead of the PV MFMAs

// Softmax weights of one tile (exp2 domain), computed a few instructions at a
// time between the MFMAs of the previous tile's P.C (whose MFMAs leave the
// issue slots free; the logits' MFMAs are busy with their own operands).  In:
// lg, the lane's 16 logits (reg j: logits row 8(j/4) + 4hf + j%4 of its head),
// row-column scaled and masked.  Out: pn, the bf16 weights p = 2^(lg - m_ref)
// as the B operand of the tile's P.C (pb once that starts), and the running
// sum of the weights as rounded.
struct Soft {
  float lg[16];
  float mx[4];
  float e[16];
  bf16x8 pb[2];  // weights of the tile whose P.C runs now
  bf16x8 pn[2];  // weights of the next tile, being computed
};

constexpr int kSoftSteps = 30;  // the schedule below, spread over the P.C steps
static_assert(kSoftSteps <= kPvSteps, "softmax schedule fits the P.C steps");

// Step s (0 <= s < kSoftSteps) of the softmax schedule.  The first tile of a
// segment sets the per-head reference m_ref (the only place where the two
// halves of a head, lanes l and l ^ 32, exchange their maxima); a later tile
// only checks its own lanes against it: a logit more than 2^kOverflowLog2
// above the reference makes the workgroup stream the segment again with the
// reference raised.
// Each result is pinned where it is computed by an empty asm that uses it:
// otherwise the compiler sinks the exponentials and conversions below the
// MFMAs, next to their use in P.C, and nothing overlaps.
__device__ __forceinline__ void soft_step(int s, Wave& w, Soft& sf, int wave) {
  if (s < 4) {
    sf.mx[s] = fmaxf(fmaxf(sf.lg[4 * s], sf.lg[4 * s + 1]), fmaxf(sf.lg[4 * s + 2], sf.lg[4 * s + 3]));
    asm volatile("" : "+v"(sf.mx[s]));
  } else if (s == 4) {
    const float mt = fmaxf(fmaxf(sf.mx[0], sf.mx[1]), fmaxf(sf.mx[2], sf.mx[3]));
    if (!w.have_ref) {  // first tile of the segment: the per-head reference
      w.m_ref = halves_max(mt);
      w.have_ref = true;
    }
    sf.mx[0] = mt;
  } else if (s == 5) {
    if (__ballot(sf.mx[0] > w.m_ref + kOverflowLog2) != 0) {
      w.m_ref = fmaxf(w.m_ref, halves_max(sf.mx[0]));
      lds_restart[wave] = 1;
    }
  } else if (s < 22) {
    // weight j, and each pair as soon as it is complete to bf16 (so that the
    // fp32 weights are not all live at once)
    const int j = s - 6;
    sf.e[j] = __builtin_amdgcn_exp2f(sf.lg[j] - w.m_ref);
    if (j & 1) {
      const int k = j >> 1;  // weights 2k, 2k + 1
      sf.pn[k >> 2][2 * (k & 3)] = (__bf16)sf.e[2 * k];
      sf.pn[k >> 2][2 * (k & 3) + 1] = (__bf16)sf.e[2 * k + 1];
      if ((k & 3) == 3) asm volatile("" : "+v"(sf.pn[k >> 2]));
    }
  } else if (s < kSoftSteps) {
    // l sums the weights as rounded for P.C, one dword (two bf16) a step: the
    // fp32 values are the dword's high half and its low half shifted up
    const int d = s - 22;
    const uint32_t u = ((const uint32_t*)&sf.pn[d >> 2])[d & 3];
    w.l_run += __uint_as_float(u << 16) + __uint_as_float(u & 0xFFFF0000u);
    asm volatile("" : "+v"(w.l_run));
  }
}

// Logits of the tile in stage S: S^T[32 tokens][32 heads] on MFMA, K-steps
// 0..3 over the 64 RoPE dims into sr, then 32 over the latent into sc (the
// A operand of step s + kQkAhead is read while step s multiplies); then the
// row-column scaling l = S_c * alpha^k + S_r (QK norm) or S_c + S_r (plain
// MLA), and the mask of a sequence's last tile.
// The logits' MFMAs as inline asm, so that their accumulators can be VGPRs:
// the compiler gives every builtin MFMA an AGPR accumulator, and with the
// AGPRs full of O^T it would move a block of O^T out and back around every
// tile.  The compiler does not see these as MFMAs, so the one hazard that
// concerns them is handled here: a VALU access to an MFMA result needs wait
// states after the MFMA (mfma_results_ready gives 24, more than the 16-pass
// case needs).  Back-to-back MFMAs on the same accumulator need none, and the
// operands come from LDS reads, which the wait counts order.
__device__ __forceinline__ void mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_next(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_results_ready(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

template <bool QKN, int S>
__device__ __forceinline__ void qk_tile(Wave& w, float* lg_out, bool last, int tail, int wave,
                                        int lane, int g) {
  const char* st = stage_buf<S>();
  const int hf = lane >> 5;
  const int m = lane & 31;
  const char* row = st + slot_token(m) * kLatRow + hf * 16;
  const char* rrow = st + kLatBytes + (32 * hf + m) * 16;
  auto qk_a = [&](int s) -> const bf16x8* {
    return (const bf16x8*)(s < kRopeSteps ? rrow + s * 1024 : row + (s - kRopeSteps) * 32);
  };
  f32x16 sc, sr;
  f32x4 ak[4];
  const float* al = (const float*)(st + kLatBytes + kRopeBytes) + g * 32 + 4 * hf;
  bf16x8 av[kQkAhead];
  bf16x8 qr[kRopeSteps];
  fence();
#pragma unroll
  for (int k = 0; k < kQkAhead; ++k) av[k] = *qk_a(k);
  const bf16x8* qrl = (const bf16x8*)(lds_qrope + (wave * kRopeSteps * 64 + lane) * 16);
#pragma unroll
  for (int k = 0; k < kRopeSteps; ++k) qr[k] = qrl[k * 64];
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) {
    fence();
    if (s == 0) mfma_first(sr, av[0], qr[0]);
    else if (s < kRopeSteps) mfma_next(sr, av[s % kQkAhead], qr[s]);
    else if (s == kRopeSteps) mfma_first(sc, av[s % kQkAhead], w.qt[0]);
    else mfma_next(sc, av[s % kQkAhead], w.qt[s - kRopeSteps]);
    if (s + kQkAhead < kQkSteps) av[s % kQkAhead] = *qk_a(s + kQkAhead);
    else if (QKN && s + kQkAhead - kQkSteps < 4) {
      const int q = s + kQkAhead - kQkSteps;  // alpha^k of the lane's tokens 8q+4hf..+3
      ak[q] = *(const f32x4*)(al + 8 * q);
    }
  }
  fence();
  mfma_results_ready(sc, sr);
  // reg j holds token 8*(j/4) + 4*hf + j%4
  if constexpr (QKN) {
#pragma unroll
    for (int j = 0; j < 16; ++j) lg_out[j] = sc[j] * ak[j >> 2][j & 3] + sr[j];
  } else {  // plain MLA: the same two sums, without the row-column scaling
#pragma unroll
    for (int j = 0; j < 16; ++j) lg_out[j] = sc[j] + sr[j];
  }
  // Only a sequence's last tile has rows to mask (tail: its rows inside the
  // sequence, wave-uniform), and the uniform test keeps the mask code off the
  // other tiles' path.
  if (last) {
    // reg j is logits row 8*(j/4) + 4*hf + j%4, i.e. token
    // slot_token(8*(j/4) + j%4) + hf; it is real iff that is below tail
    const int thr = tail - hf;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (slot_token(8 * (j >> 2) + (j & 3)) >= thr) lg_out[j] = -INFINITY;
  }
}

// O^T[512 dims][32 heads] += C^T . P^T over the tile in stage S, with B = P
// straight from the softmax registers (token order permuted to match) and
// A = C^T from ds_read_b64_tr_b16: for step k = 16*ks + mb, lane (in its
// 16-lane group) reads the token of logits row 16*ks + 4*hf + (s16>>2), which
// is latent row 16*ks + 4*(s16>>2) + hf (row + 2 for logits rows 8 further
// on), 4 dims at 32*mb + 16*dblk + 4*(s16&3).  With SOFT, the softmax of the
// next tile (sf.lg -> sf.pn) runs between the MFMAs.
template <bool SOFT, int S>
__device__ __forceinline__ void pv_tile(Wave& w, Soft& sf, int wave, int lane) {
  const char* st = stage_buf<S>();
  const int hf = lane >> 5;
  const int s16 = lane & 15, dblk = (lane >> 4) & 1;
  const char* pvb = st + (4 * (s16 >> 2) + hf) * kLatRow + 32 * dblk + 8 * (s16 & 3);
  auto pv_a = [&](int k) -> const char* {
    return pvb + (16 * (k / (kR / 32))) * kLatRow + 64 * (k % (kR / 32));
  };
  bf16x4 plo[kPvAhead], phi[kPvAhead];
  fence();
#pragma unroll
  for (int k = 0; k < kPvAhead; ++k) {
    plo[k] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pv_a(k)));
    phi[k] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pv_a(k) + 2 * kLatRow));
  }
#pragma unroll
  for (int k = 0; k < kPvSteps; ++k) {
    fence();
    const int slot = k % kPvAhead;
    const bf16x8 a8 = {plo[slot][0], plo[slot][1], plo[slot][2], plo[slot][3],
                       phi[slot][0], phi[slot][1], phi[slot][2], phi[slot][3]};
    const int mb = k % (kR / 32);
    w.O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, sf.pb[k / (kR / 32)], w.O[mb], 0, 0, 0);
    if (k + kPvAhead < kPvSteps) {
      plo[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(QK_LDS(bf16x4, pv_a(k + kPvAhead)));
      phi[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          QK_LDS(bf16x4, pv_a(k + kPvAhead) + 2 * kLatRow));
    }
    if constexpr (SOFT) {
      if (k < kSoftSteps) soft_step(k, w, sf, wave);
    }
  }
  fence();
}

// One step of the software pipeline over a segment's nt tiles, tile i in
// stage i % 3 (SP), tile i + 1 in SQ, the stage of tile i - 1 free (SN):
//   wait for tile i + 1 and synchronise the workgroup (every wave is past
//   tile i - 1, so stage SN is free), prefetch tile i + 2 into SN; the logits
//   of tile i + 1 on MFMA; then the P.C of tile i with the softmax of tile
//   i + 1 between its MFMAs.  pb holds the weights of tile i on entry and of
//   tile i + 1 on exit.  The prefetch of tile 2 is issued by the segment's
//   first step (stage 2 is free from the start), so step 0 does not issue
//   one.
template <bool QKN, int NW, int SP, int SQ, int SN>
__device__ __forceinline__ void pipe_step(Wave& w, Soft& sf, const Seq& sq, const Paging& pg,
                                          int G, int tile0, int i, int nt, int wave, int lane,
                                          int g) {
  wait_vmcnt<0>();
  block_sync();
  if (i >= 1 && i + 2 < nt) issue_tile<QKN, NW, SN>(sq, pg, G, tile0 + i + 2, wave, lane);
  if (i + 1 < nt) {
    const int t = tile0 + i + 1;
    const bool last = t == sq.last_tile;
    const int tail = last ? __builtin_amdgcn_readfirstlane(sq.L - t * kTile) : kTile;
    qk_tile<QKN, SQ>(w, sf.lg, last, tail, wave, lane, g);
  } else {
    // no next tile: its softmax sees only masked logits, so it adds nothing
    // (one P.C code path for all steps keeps the accumulators in place)
#pragma unroll
    for (int j = 0; j < 16; ++j) sf.lg[j] = -INFINITY;
  }
  pv_tile<true, SP>(w, sf, wave, lane);
  sf.pb[0] = sf.pn[0];
  sf.pb[1] = sf.pn[1];
}

template <bool QKN, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(Args a) {
  // Contiguous caches get their own instantiation, in which the block-table
  // test folds away (a runtime flag would be one more value held in registers
  // across the segment loop).
  Paging pg = a.pg;
  if constexpr (!PAGED) pg.bt = nullptr;
  // The tile prefix takes LDS offset 0 (largest alignment is placed first): a
  // stage buffer at offset 0 loses the alias information that lets its reads
  // run ahead of the loads in flight into the other stages.
  __shared__ __attribute__((aligned(2048))) int P[kMaxBatch + 1];
  if (threadIdx.x < 4) lds_restart[threadIdx.x] = 0;
  build_tile_prefix(a.seq_lens, a.B, a.s_q, pg.capacity(), P);
  if (blockIdx.x == 0)  // the merge reads the prefix instead of rebuilding it per block
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.plan[i] = P[i];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5;        // which half of the 64 lanes
  const int n = lane & 31;         // head column within the wave
  const int head = wave * 32 + n;  // head index in the layer
  const int g = (head * a.G) / a.H;
  const int64_t N = __builtin_amdgcn_readfirstlane(P[a.B]);
  const int p = plan_wg(blockIdx.x, a.n_wg);
  int64_t x = wg_start(p, N, a.n_wg);
  const int64_t e = wg_start(p + 1, N, a.n_wg);
  bool first_seg = true;
  Wave w;

  while (x < e) {
    // b: virtual sequence (query row b % s_q of cache b / s_q)
    const int b = __builtin_amdgcn_readfirstlane(seq_of(P, a.B, x));
    Seq sq;
    sq.L = __builtin_amdgcn_readfirstlane(virt_len(a.seq_lens, b, a.s_q, pg.capacity()));
    const int64_t s0 = __builtin_amdgcn_readfirstlane(P[b]);
    const int64_t s1 = __builtin_amdgcn_readfirstlane(P[b + 1]);
    const int64_t seg_end = e < s1 ? e : s1;
    const int tile0 = (int)(x - s0);
    const int nt = (int)(seg_end - x);
    sq.cb = b / a.s_q;
    sq.last_tile = (int)(s1 - s0) - 1;
    sq.lat = (const char*)a.lat;
    sq.rope = (const char*)a.rope;
    sq.alpha = QKN ? (const char*)a.alpha : nullptr;

    // The segment's loads, in the order the first tile's logits need them:
    // the RoPE query (straight into LDS: its operand-order rows are the LDS
    // layout) and tile 0; then q~ into registers (operand order: each load
    // reads the wave's 1 KB of one K-step); then tile 1.  Loads complete in
    // order, so the first logits wait only for the first group, and the q~
    // loads land while the MFMAs run (the compiler waits for each as it is
    // used).  The fences keep the groups in this order.
    {
      const __amdgpu_buffer_rsrc_t qr_rsrc = tile_rsrc(
          a.q_rope + qop_index(b, a.H, kDr, wave * 32, 0), (kDr / 16) * 64 * 16);
#pragma unroll
      for (int s = 0; s < kDr / 16; ++s)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            qr_rsrc, QK_LDS(void, lds_qrope + (wave * (kDr / 16) + s) * 1024), 16, lane << 4,
            s * 1024, 0, 0);
    }
    issue_tile<QKN, NW, 0>(sq, pg, a.G, tile0, wave, lane);
    fence();
    {
      // scalar base (the wave's block) plus a lane offset recomputed here, so
      // that no per-lane address is kept, or spilled, across the segments
      const char* qbase = (const char*)(a.q_tilde + qop_index(b, a.H, kR, wave * 32, 0));
      uint32_t ln16;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
                   "v_lshlrev_b32 %0, 4, %0" : "=v"(ln16));
#pragma unroll
      for (int s = 0; s < kR / 16; ++s) w.qt[s] = *(const bf16x8*)(qbase + s * 1024 + ln16);
    }
    fence();
    if (nt > 1) issue_tile<QKN, NW, 1>(sq, pg, a.G, tile0 + 1, wave, lane);
    bool q_in_flight = true;
    w.m_ref = -INFINITY;
    w.have_ref = false;
    for (;;) {  // one pass over the segment; repeated only if a logit overflows the reference
#pragma unroll
      for (int ii = 0; ii < kR / 32; ++ii)
#pragma unroll
        for (int j = 0; j < 16; ++j) w.O[ii][j] = 0.f;
      w.l_run = 0.f;
      Soft sf;
      {  // the first tile's logits; stage 2 is free, so tile 2 goes out now
        // Wait for tile 0 (and the RoPE query): on a segment's first pass the
        // q~ loads and tile 1 may still be in flight behind them.
        constexpr int kQtLoads = kR / 16;
        if (!q_in_flight) wait_vmcnt<0>();
        else if (nt > 1) {
          // (the counter holds at most 63: with one wavefront, 72 loads follow
          // tile 0, and waiting for nine more of them costs nothing that matters)
          constexpr int kAfter = kQtLoads + TileLoads<QKN, NW>::total;
          wait_vmcnt<(kAfter < 64 ? kAfter : 63)>();
        }
        else wait_vmcnt<kQtLoads>();
        q_in_flight = false;
        block_sync();
        if (nt > 2) issue_tile<QKN, NW, 2>(sq, pg, a.G, tile0 + 2, wave, lane);
        const bool last = tile0 == sq.last_tile;
        const int tail = last ? __builtin_amdgcn_readfirstlane(sq.L - tile0 * kTile) : kTile;
        qk_tile<QKN, 0>(w, sf.lg, last, tail, wave, lane, g);
#pragma unroll
        for (int s = 0; s < kSoftSteps; ++s) soft_step(s, w, sf, wave);
        sf.pb[0] = sf.pn[0];
        sf.pb[1] = sf.pn[1];
      }
      for (int i = 0; i < nt; i += kStages) {
        pipe_step<QKN, NW, 0, 1, 2>(w, sf, sq, pg, a.G, tile0, i, nt, wave, lane, g);
        if (i + 1 < nt) pipe_step<QKN, NW, 1, 2, 0>(w, sf, sq, pg, a.G, tile0, i + 1, nt, wave, lane, g);
        if (i + 2 < nt) pipe_step<QKN, NW, 2, 0, 1>(w, sf, sq, pg, a.G, tile0, i + 2, nt, wave, lane, g);
      }
      block_sync();
      if (!(lds_restart[0] | lds_restart[1] | lds_restart[2] | lds_restart[3])) break;
      // A logit exceeded the reference by more than 2^kOverflowLog2: stream the
      // segment again with the raised reference (exact; never taken for
      // normalised logits).
      block_sync();
      if (lane_here() == 0) lds_restart[wave] = 0;
      issue_tile<QKN, NW, 0>(sq, pg, a.G, tile0, wave, lane);
      if (nt > 1) issue_tile<QKN, NW, 1>(sq, pg, a.G, tile0 + 1, wave, lane);
    }
    // ---- segment epilogue ----
    // The accumulator holds, in lane (head 32 wave + lane % 32, hf = lane / 32)
    // and register i of block mb, latent dim 32 mb + 8 (i / 4) + 4 hf + i % 4.
    // It goes out through LDS, so that each store writes whole rows: the
    // stage buffers are idle here (every wave is past the segment's last
    // tile), and wave w transposes through its own 32-row region of them,
    // one round of kEpiDims dims at a time.
    const float l_tot = halves_sum(w.l_run);
    const float m_run = w.m_ref;
    const bool complete = (x == s0) && (seg_end == s1);
    // The lane values are re-derived here, so that the epilogue's addresses
    // are formed here rather than kept live across the tile loop.
    const int ln = lane_here();
    const int en = ln & 31, ehf = ln >> 5;
    const int ehead = wave * 32 + en;
    char* region = (wave >> 1 == 0 ? stage_buf<0>() : stage_buf<1>()) + (wave & 1) * kEpiRegion;
    // Each round reads its 16 LDS rows kEpiBatch at a time into registers
    // before their stores, so the reads overlap and a store does not wait on
    // the read just before it.  A store's address is the wave's row block
    // (scalar) plus a 32-bit lane offset.
    if (complete) {  // normalised o_lat, fp32 rows of 2 KB: four rounds of 128 dims
      const float inv = 1.0f / l_tot;
      char* out = (char*)(a.o_lat + (size_t)b * a.H * kR) + (size_t)(wave * 32) * kR * 4;
      const uint32_t lane_off = (uint32_t)ehf * (kR * 4) + (uint32_t)en * 16;
#pragma unroll
      for (int rnd = 0; rnd < kR / 128; ++rnd) {
        fence();  // one round at a time: its accumulator reads are not hoisted
#pragma unroll
        for (int mbl = 0; mbl < 4; ++mbl)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int mb = rnd * 4 + mbl;
            const f32x4 v = {w.O[mb][4 * q] * inv, w.O[mb][4 * q + 1] * inv,
                             w.O[mb][4 * q + 2] * inv, w.O[mb][4 * q + 3] * inv};
            *(f32x4*)(region + en * kEpiRow + (32 * mbl + 8 * q + 4 * ehf) * 4) = v;
            fence();  // a few accumulator registers in flight at a time
          }
        fence();
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += kEpiBatch) {
          uint4 rows[kEpiBatch];
#pragma unroll
          for (int it = 0; it < kEpiBatch; ++it)
            rows[it] = *(const uint4*)(region + (2 * (i0 + it) + ehf) * kEpiRow + en * 16);
#pragma unroll
          for (int it = 0; it < kEpiBatch; ++it)
            *(uint4*)(out + (size_t)(2 * (i0 + it)) * kR * 4 + rnd * 512 + lane_off) = rows[it];
          __builtin_amdgcn_sched_group_barrier(0x100, kEpiBatch, 0);  // the LDS reads first,
          __builtin_amdgcn_sched_group_barrier(0x040, kEpiBatch, 0);  // then the stores
        }
      }
      if (ehf == 0 && a.lse) a.lse[(size_t)b * a.H + ehead] = (m_run + log2f(l_tot)) * kLn2;
    } else {  // partial: m, l and the unnormalised O in bf16, rows of 1 KB: two rounds of 256 dims
      const int slot = first_seg ? 0 : 1;
      char* sp = a.part + ((size_t)p * kSlotsPerWg + slot) * kPartialSlotBytes(a.H, kR);
      if (ehf == 0) {
        ((float*)sp)[ehead] = m_run;
        ((float*)sp)[a.H + ehead] = l_tot;
      }
      char* Op = sp + (size_t)a.H * 8 + (size_t)(wave * 32) * kR * 2;
      const uint32_t lane_off = (uint32_t)ehf * (kR * 2) + (uint32_t)en * 16;
#pragma unroll
      for (int rnd = 0; rnd < kR / 256; ++rnd) {
        fence();  // one round at a time: its accumulator reads are not hoisted
#pragma unroll
        for (int mbl = 0; mbl < 8; ++mbl)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int mb = rnd * 8 + mbl;
            bf16x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (__bf16)w.O[mb][4 * q + j];
            *(bf16x4*)(region + en * kEpiRow + (32 * mbl + 8 * q + 4 * ehf) * 2) = v;
            fence();  // a few accumulator registers in flight at a time
          }
        fence();
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += kEpiBatch) {
          uint4 rows[kEpiBatch];
#pragma unroll
          for (int it = 0; it < kEpiBatch; ++it)
            rows[it] = *(const uint4*)(region + (2 * (i0 + it) + ehf) * kEpiRow + en * 16);
#pragma unroll
          for (int it = 0; it < kEpiBatch; ++it)
            *(uint4*)(Op + (size_t)(2 * (i0 + it)) * kR * 2 + rnd * 512 + lane_off) = rows[it];
          __builtin_amdgcn_sched_group_barrier(0x100, kEpiBatch, 0);  // the LDS reads first,
          __builtin_amdgcn_sched_group_barrier(0x040, kEpiBatch, 0);  // then the stores
        }
      }
    }
    first_seg = false;
    x = seg_end;
    block_sync();  // all waves done with the stage buffers before the next segment
  }
}

}  // namespace

hipError_t launch_decode_mfma(const Cfg& c, int batch, int s_q, const int32_t* seq_lens,
                              const Paging& pg, const void* lat, const void* rope,
                              const float* alpha, const WsLayout& ws, void* workspace, int n_wg,
                              float* o_lat, float* lse, hipStream_t s) {
  char* wsb = (char*)workspace;
  Args a;
  a.seq_lens = seq_lens;
  a.B = batch * s_q;
  a.s_q = s_q;
  a.H = c.H;
  a.G = c.G;
  a.pg = pg;
  a.n_wg = n_wg;
  a.lat = (const uint16_t*)lat;
  a.rope = (const uint16_t*)rope;
  a.alpha = alpha;
  a.q_tilde = (const uint16_t*)(wsb + ws.q_tilde);
  a.q_rope = (const uint16_t*)(wsb + ws.q_rope);
  a.part = wsb + ws.partials;
  a.plan = (int32_t*)(wsb + ws.plan);
  a.o_lat = o_lat;
  a.lse = lse;
  const int nw = c.H / 32;
  const bool paged = pg.bt != nullptr;
  dim3 grid(n_wg), block(nw * 64);
  void (*k)(Args) = nullptr;
  if (c.qk_norm) {
    if (nw == 4) k = paged ? decode_mfma_kernel<true, 4, true> : decode_mfma_kernel<true, 4, false>;
    else if (nw == 2) k = paged ? decode_mfma_kernel<true, 2, true> : decode_mfma_kernel<true, 2, false>;
    else if (nw == 1) k = paged ? decode_mfma_kernel<true, 1, true> : decode_mfma_kernel<true, 1, false>;
  } else {
    if (nw == 4) k = paged ? decode_mfma_kernel<false, 4, true> : decode_mfma_kernel<false, 4, false>;
    else if (nw == 2) k = paged ? decode_mfma_kernel<false, 2, true> : decode_mfma_kernel<false, 2, false>;
    else if (nw == 1) k = paged ? decode_mfma_kernel<false, 1, true> : decode_mfma_kernel<false, 1, false>;
  }
  if (!k) return hipErrorInvalidValue;
  return launch_kernel(k, grid, block, s, a);
}

}  // namespace qkmla
