/*
 * qkmla.h -- C ABI of the MI355X (gfx950) QK-Normed MLA latent decode library.
 *
 * The method ("QK-Normed MLA: QK normalization without full key caching"):
 * post-projection QK RMSNorm folded into MLA's absorbed latent decode path.
 * RMSNorm(z) = z * gamma / S(z) splits into a static weight gamma and a dynamic
 * scalar S(z) (technical summary, Methodology: RMSNorm decomposition).  The
 * static weights gamma_q, gamma_k fold into the query-side latent projection
 * (Methodology: Static Weight Absorption); the key statistic becomes one
 * inverse-RMS scalar alpha^k per token and KV group, kept in a small cache
 * beside the latent cache (Methodology: Dynamic Scalar Caching, Cache Layout).
 * Decode logits are (q~ . c_t) * alpha^q * alpha^k (Methodology: decode-logit
 * formula) plus a separately RMS-normed RoPE term (Methodology: Blockwise
 * Normalization), then softmax, latent-weighted accumulation and the V
 * up-projection.  The abstract states the absorbed form equals explicit
 * post-projection QK RMSNorm in exact arithmetic.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument named as "device" is device memory (hipMalloc or a
 *    torch CUDA tensor) on the current HIP device, row-major and contiguous,
 *    aligned to its element size.  qkmla_decode in bf16 additionally needs
 *    16-byte alignment of q_c, q_rope, w_qabs, both caches and o_lat (rows are
 *    read as 16-byte vectors); every workspace is 16-byte aligned.
 *  - Every buffer and the stream are owned by the caller.  The library never
 *    allocates, frees or synchronises; all work is enqueued on `stream`
 *    (a hipStream_t passed as void*, NULL = the default stream) and the call
 *    returns without waiting.
 *  - Return value: a qkmla_status.  On a non-zero status nothing was enqueued;
 *    qkmla_last_error() (thread-local) describes the failure.
 *  - Data errors that only the device can see (a sequence length outside
 *    [1, cache_capacity], an append position outside the cache) are reported by
 *    OR-ing QKMLA_DEV_* bits into `*status` (device int32, may be NULL).  The
 *    caller clears it.  The affected sequence gets no cache writes (append) or
 *    an all-zero output with lse = -inf (decode).
 *  - batch == 0 (packed training: no sequences or no tokens) is a valid no-op
 *    returning QKMLA_OK.
 *
 * Readings of points the pages leave open (the oracle makes the same ones):
 *  - S(z) = sqrt(mean(z^2) + eps), eps inside the square root.
 *  - gamma_q, gamma_k are [head_dim] vectors shared by all heads and groups;
 *    the RoPE part has its own gamma_q_rope, gamma_k_rope of [rope_dim].
 *  - One RoPE key per token shared by all heads, RMS-normalised and then
 *    rotated; RoPE rotates interleaved pairs (2i, 2i+1) by p*base^(-2i/rope_dim);
 *    the key at cache row t has position t, the query position seq_len-1.
 *  - logit = softmax_scale * (content + rope); the alpha factors scale only the
 *    content term.  Head h belongs to KV group floor(h*G/H).
 */
#ifndef QKMLA_H_
#define QKMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKMLA_ABI_VERSION 8

typedef enum {
  QKMLA_OK = 0,
  QKMLA_ERR_INVALID_ARG = 1,    /* null / misaligned pointer, bad sizes, H % G != 0, odd rope_dim */
  QKMLA_ERR_UNSUPPORTED = 2,    /* valid but not compiled (see qkmla_config) */
  QKMLA_ERR_WORKSPACE = 3,      /* workspace smaller than qkmla_decode_workspace_size() */
  QKMLA_ERR_HIP = 4             /* a HIP launch failed; message from the HIP runtime */
} qkmla_status;

typedef enum { QKMLA_F32 = 0, QKMLA_BF16 = 1 } qkmla_dtype;

/* Device-side data-error bits OR-ed into *status. */
#define QKMLA_DEV_BAD_SEQ_LEN 1   /* decode: seq_len outside [1, cache_capacity];
                                     packed training: cu_seqlens breaks its rules */
#define QKMLA_DEV_BAD_POSITION 2  /* append: position < 0 or position + n_new > cache_capacity */
#define QKMLA_DEV_BAD_PAGE 4      /* paged caches: a needed block-table entry is outside [0, num_pages) */

/*
 * Layer shape and mode.
 *   n_heads H, n_groups G (H % G == 0), latent_rank r, head_dim d_c,
 *   rope_dim d_r (even), v_head_dim d_v.
 *   dtype: storage type of the latent and RoPE caches, queries, absorbed query
 *     weights and W^UV.  The alpha cache, W^UK, all gammas and every output are
 *     float32.  All arithmetic accumulates in float32.
 *     QKMLA_F32: any shape with r <= 1024, d_c <= 1024, d_r <= 256, d_v <= 1024.
 *     QKMLA_BF16: r = 512, d_r = 64, H in {32, 64, 128}, H/G = 16, d_c a multiple
 *     of 32 up to 256 (the DeepSeek-V3-like MLA layer); d_v <= 1024.
 *   qk_norm: 1 = QK-Normed MLA; 0 = plain MLA (no gammas, no alpha, no RoPE
 *     norm) -- the same kernels with the normalisation compiled out.
 *   eps: RMSNorm epsilon (>= 0).
 *   softmax_scale: tau; <= 0 selects 1/sqrt(d_c + d_r).
 *   rope_base: RoPE base (> 0), e.g. 10000.
 */
typedef struct {
  int32_t n_heads, n_groups, latent_rank, head_dim, rope_dim, v_head_dim;
  int32_t dtype;
  int32_t qk_norm;
  float eps;
  float softmax_scale;
  float rope_base;
} qkmla_config;

/*
 * Static weight absorption (Methodology: Static Weight Absorption).
 *   w_uk     device float [G][r][d_c]   key up-projection W^UK (k_g = c W^UK_g)
 *   gamma_q  device float [d_c]         query RMSNorm weight (ignored if !qk_norm)
 *   gamma_k  device float [d_c]         key RMSNorm weight   (ignored if !qk_norm)
 *   w_qabs   device dtype [G][r][d_c]   out: W~_g^T, element (g,i,j) =
 *            gamma_q[j]*gamma_k[j]*W^UK[g][i][j] rounded to dtype (W^UK itself
 *            if !qk_norm).  This is diag(gamma_q gamma_k)(W^UK_g)^T stored with
 *            d_c innermost so the query projection q~ = q^C W~_g reads rows.
 * One-time; off the per-step clock.
 */
int qkmla_absorb_weights(const qkmla_config* cfg, const float* w_uk, const float* gamma_q,
                         const float* gamma_k, void* w_qabs, void* stream);

/*
 * Append n_new tokens to every sequence of the batch (Methodology: Dynamic
 * Scalar Caching, Cache Layout, Blockwise Normalization).  For sequence b and
 * i < n_new the row t = positions[b] + i of each cache is written:
 *   latent_cache[b][t][:] = c_new[b][i][:]                       (copy)
 *   alpha_cache[b][t][g]  = 1/sqrt(mean_j (c_new W^UK_g)_j^2 + eps) for each g,
 *                           computed in float32 from the stored latent and
 *                           float32 W^UK (only if qk_norm)
 *   rope_cache[b][t][:]   = RoPE_t(k_rope_new * gamma_k_rope / S(k_rope_new))
 *                           (without the norm if !qk_norm), rounded to dtype.
 *   c_new          device dtype [B][n_new][r]
 *   k_rope_new     device dtype [B][n_new][d_r]    raw RoPE key (before norm/RoPE)
 *   w_uk           device float [G][r][d_c]        (unused if !qk_norm)
 *   gamma_k_rope   device float [d_r]              (unused if !qk_norm)
 *   positions      device int32 [B]                first cache row per sequence
 *   cache_capacity L_cap: rows per sequence in each cache
 *   latent_cache   device dtype [B][L_cap][r]
 *   rope_cache     device dtype [B][L_cap][d_r]
 *   alpha_cache    device float [B][L_cap][G]      (may be NULL if !qk_norm)
 *   status         device int32, nullable: QKMLA_DEV_BAD_POSITION on a bad row
 */
int qkmla_append(const qkmla_config* cfg, int32_t batch, int32_t n_new, const void* c_new,
                 const void* k_rope_new, const float* w_uk, const float* gamma_k_rope,
                 const int32_t* positions, int32_t cache_capacity, void* latent_cache,
                 void* rope_cache, float* alpha_cache, int32_t* status, void* stream);

/*
 * Bytes of device workspace qkmla_decode needs for this batch and length bound
 * (query staging, split partials and plan data).  0 on invalid arguments.
 */
size_t qkmla_decode_workspace_size(const qkmla_config* cfg, int32_t batch, int32_t max_seq_len);

/*
 * One decode step (s_q = 1) over the latent, RoPE and alpha caches: split-KV
 * flash-decoding.  Per sequence b (L_b = seq_lens[b]), head h, g = g(h):
 *   alpha^q_h = 1/S(q_c[b][h]),  q~_h = q_c[b][h] W~_g,
 *   q^R_h = RoPE_{L_b-1}(q_rope[b][h] * gamma_q_rope / S(q_rope[b][h])),
 *   logit_t = tau * ((q~_h . c_t) alpha^q_h alpha_cache[b][t][g] + q^R_h . k^R_t),
 *   p = softmax over t < L_b,
 *   o_lat[b][h][:] = sum_t p_t c_t,  lse[b][h] = log sum_t exp(logit_t).
 * (Plain MLA if !qk_norm: no alpha, no norms.)
 *   q_c          device dtype [B][H][d_c]    content query (projected, before norm)
 *   q_rope       device dtype [B][H][d_r]    RoPE query (before norm and RoPE)
 *   w_qabs       device dtype [G][r][d_c]    from qkmla_absorb_weights
 *   gamma_q_rope device float [d_r]          (unused if !qk_norm)
 *   latent_cache, rope_cache, alpha_cache    as written by qkmla_append
 *   seq_lens     device int32 [B]            L_b, valid range [1, L_cap]
 *   cache_capacity L_cap;  max_seq_len: host upper bound on every L_b (<= L_cap)
 *   workspace    device, >= qkmla_decode_workspace_size(cfg, batch, max_seq_len) bytes
 *   o_lat        device float [B][H][r]      out
 *   lse          device float [B][H]         out, nullable (natural log)
 *   status       device int32, nullable      QKMLA_DEV_BAD_SEQ_LEN
 */
int qkmla_decode(const qkmla_config* cfg, int32_t batch, const void* q_c, const void* q_rope,
                 const void* w_qabs, const float* gamma_q_rope, const void* latent_cache,
                 const void* rope_cache, const float* alpha_cache, const int32_t* seq_lens,
                 int32_t cache_capacity, int32_t max_seq_len, void* workspace,
                 size_t workspace_bytes, float* o_lat, float* lse, int32_t* status,
                 void* stream);

/*
 * qkmla_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and outputs as qkmla_decode, without the workspace: the library
 * uses its own scratch array of QKMLA_NOALLOC_SCRATCH_BYTES per GPU (static
 * device memory, held by every GPU the library runs on until the process
 * ends; its address is looked up once per device on the first call there).
 * The call allocates nothing, neither device nor host memory.
 *   Limit: a call whose qkmla_decode_workspace_size(cfg, batch, max_seq_len)
 *   exceeds QKMLA_NOALLOC_SCRATCH_BYTES returns QKMLA_ERR_WORKSPACE (e.g. the
 *   bf16 128-head layer fits up to a few hundred sequences); nothing is
 *   enqueued.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap on
 *   one GPU (on different streams, or from different host threads without
 *   ordering) race and their outputs are undefined.  Calls enqueued in order
 *   on one stream are safe.  Nothing in the scratch needs to start at zero.
 */
#define QKMLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int qkmla_decode_noalloc(const qkmla_config* cfg, int32_t batch, const void* q_c,
                         const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                         const void* latent_cache, const void* rope_cache,
                         const float* alpha_cache, const int32_t* seq_lens,
                         int32_t cache_capacity, int32_t max_seq_len, float* o_lat, float* lse,
                         int32_t* status, void* stream);

/*
 * Decode of s_q query rows per sequence (multi-token prediction,
 * speculative verification), causal over the cache.  The pages' decode logit
 * carries a query index i ("QK-Normed MLA: QK normalization without full key
 * caching", technical summary, Methodology: decode-logit formula); here row i
 * of sequence b is the token at position P_i = L_b - s_q + i, whose latent,
 * RoPE and alpha rows are already in the cache (appended before the call):
 * it attends cache rows 0..P_i and its RoPE query is rotated by P_i.  Each
 * row is exactly the s_q = 1 decode of qkmla_decode with seq_len P_i + 1.
 *   q_c     device dtype [B][s_q][H][d_c];  q_rope device dtype [B][s_q][H][d_r]
 *   seq_lens device int32 [B]: L_b, counting the s_q new tokens
 *   workspace >= qkmla_decode_workspace_size(cfg, batch * s_q, max_seq_len)
 *   o_lat   device float [B][s_q][H][r] out;  lse device float [B][s_q][H], nullable
 *   other arguments as for qkmla_decode.
 * A row whose prefix length P_i + 1 is outside [1, L_cap] (L_b < s_q - i, or
 * L_b invalid) gets zeros, lse = -inf and sets QKMLA_DEV_BAD_SEQ_LEN.
 * batch * s_q must not exceed 4096 (QKMLA_ERR_UNSUPPORTED); s_q < 1 is
 * QKMLA_ERR_INVALID_ARG.  qkmla_decode is this call with s_q = 1.
 */
int qkmla_decode_multi(const qkmla_config* cfg, int32_t batch, int32_t s_q, const void* q_c,
                       const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                       const void* latent_cache, const void* rope_cache, const float* alpha_cache,
                       const int32_t* seq_lens, int32_t cache_capacity, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                       int32_t* status, void* stream);

/*
 * Paged caches.  The pages lay the caches out as one latent row, one RoPE row
 * and G alpha scalars per cached token (Methodology: Cache Layout) and say
 * nothing of how rows are placed; a serving cache keeps them in a shared pool
 * of fixed-size pages with a block table per sequence.  Here row t of
 * sequence b lives at pool row
 *   block_table[b][t / page_size] * page_size + t % page_size
 * of each of the three pools, so the contiguous layout of qkmla_append /
 * qkmla_decode is the special case page_size = L_cap, block_table[b][0] = b.
 *   block_table  device int32 [B][max_blocks]; entries in [0, num_pages)
 *   max_blocks   blocks per sequence; the capacity L_cap = max_blocks*page_size
 *   page_size    rows per page (>= 1; bf16 decode needs a multiple of 32, the
 *                split-KV token tile, else QKMLA_ERR_UNSUPPORTED)
 *   num_pages    pages in each pool
 *   pools        latent device dtype [num_pages*page_size][r],
 *                rope   device dtype [num_pages*page_size][d_r],
 *                alpha  device float [num_pages*page_size][G]
 * The caller owns the table and the pools.  An entry that a call needs and
 * that is outside [0, num_pages) sets QKMLA_DEV_BAD_PAGE: append skips that
 * row; decode reads page 0 in its place, so that row's output is undefined.
 */
typedef struct {
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t page_size;
  int32_t num_pages;
} qkmla_pages;

/* qkmla_append into paged pools: as qkmla_append with cache_capacity =
 * max_blocks * page_size and rows placed by the block table. */
int qkmla_append_paged(const qkmla_config* cfg, int32_t batch, int32_t n_new, const void* c_new,
                       const void* k_rope_new, const float* w_uk, const float* gamma_k_rope,
                       const int32_t* positions, const qkmla_pages* pages, void* latent_pool,
                       void* rope_pool, float* alpha_pool, int32_t* status, void* stream);

/* qkmla_decode_multi over paged pools: as qkmla_decode_multi with
 * cache_capacity = max_blocks * page_size and rows read through the block
 * table.  Same outputs, to the rounding of identical arithmetic, as the
 * contiguous call over the same rows. */
int qkmla_decode_paged(const qkmla_config* cfg, int32_t batch, int32_t s_q, const void* q_c,
                       const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                       const void* latent_pool, const void* rope_pool, const float* alpha_pool,
                       const int32_t* seq_lens, const qkmla_pages* pages, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                       int32_t* status, void* stream);

/*
 * V up-projection: out[b][h][:] = o_lat[b][h][:] W^UV_{g(h)}.
 *   o_lat device float [B][H][r];  w_uv device dtype [G][r][d_v];
 *   out   device float [B][H][d_v].
 * Pointers must be aligned to their element size; for bf16 with 16 heads per
 * group, r a multiple of 128 and d_v of 16 (the MFMA kernel, which reads
 * 16-byte vectors) o_lat and w_uv must be 16-byte aligned.  A violation
 * returns QKMLA_ERR_INVALID_ARG before anything is launched.
 */
int qkmla_out_proj(const qkmla_config* cfg, int32_t batch, const float* o_lat, const void* w_uv,
                   float* out, void* stream);

/*
 * Training and prefill in the explicit form (the form the pages train with:
 * technical summary, Results; Methodology: RMSNorm decomposition, Blockwise
 * Normalization).  `batch` sequences of `seq_len` tokens each; token i of a
 * sequence sits at position i and attends tokens 0..i of its own sequence.
 * Per token i, head h, g = g(h):
 *   k_{j,g} = c_j W^UK_g (materialised),  k^ = k * gamma_k / S(k),
 *   q^ = q_c * gamma_q / S(q_c),
 *   q^R, k^R: RMS-normalised with gamma_q_rope / gamma_k_rope, rotated by
 *             their own position (one RoPE key per token, shared by all heads),
 *   logit_ij = tau (q^_i . k^_j + q^R_i . k^R_j),  j <= i,
 *   o[b][i][h] = sum_j softmax_j(logit) c_j W^UV_g,  lse = log sum_j exp(logit).
 * (Plain MLA if !qk_norm: no norms, gammas unused, their gradients zero.)
 * Shapes: any layer with d_c, d_v <= 256, r <= 1024, d_r <= 256, either
 * dtype; the bf16 decode restrictions do not apply here.
 * Arithmetic: fp32 throughout, except for the bf16 layer with 16 heads per
 * group, d_c + d_r = 192 and d_v = 128, whose attention and projections run
 * on MFMA with bf16 operands (normalised queries and keys, values, softmax
 * weights, their gradients, W^UK as a bf16 pair) and fp32 accumulation.
 * The workspace is scratch for one call; the backward recomputes what it
 * needs from the inputs, so no state passes between the two calls except
 * o and lse.
 */
typedef struct {
  const void* c;       /* device dtype [B][T][r]       latents */
  const void* q_c;     /* device dtype [B][T][H][d_c]  content queries (projected, before norm) */
  const void* q_rope;  /* device dtype [B][T][H][d_r]  RoPE queries (before norm and RoPE) */
  const void* k_rope;  /* device dtype [B][T][d_r]     RoPE keys (before norm and RoPE) */
  const float* w_uk;   /* device float [G][r][d_c] */
  const void* w_uv;    /* device dtype [G][r][d_v] */
  const float* gamma_q;      /* device float [d_c] (unused if !qk_norm) */
  const float* gamma_k;      /* device float [d_c] */
  const float* gamma_q_rope; /* device float [d_r] */
  const float* gamma_k_rope; /* device float [d_r] */
} qkmla_train_inputs;

/* Gradients of sum(o * d_o) with respect to every input: device float
 * arrays, each of its input's shape, all required.  Every element is
 * written (no accumulation into existing values). */
typedef struct {
  float *d_c, *d_q_c, *d_q_rope, *d_k_rope, *d_w_uk, *d_w_uv;
  float *d_gamma_q, *d_gamma_k, *d_gamma_q_rope, *d_gamma_k_rope;
} qkmla_train_grads;

/* Workspace bytes for qkmla_train_backward (enough for the forward too);
 * 0 on invalid arguments. */
size_t qkmla_train_workspace_size(const qkmla_config* cfg, int32_t batch, int32_t seq_len);

/* Forward: o device float [B][T][H][d_v], lse device float [B][T][H]
 * (natural log; the backward needs it). */
int qkmla_train_forward(const qkmla_config* cfg, int32_t batch, int32_t seq_len,
                        const qkmla_train_inputs* inputs, void* workspace, size_t workspace_bytes,
                        float* o, float* lse, void* stream);

/* Backward of sum(o * d_o): o and lse as the forward wrote them, d_o device
 * float [B][T][H][d_v]. */
int qkmla_train_backward(const qkmla_config* cfg, int32_t batch, int32_t seq_len,
                         const qkmla_train_inputs* inputs, const float* o, const float* lse,
                         const float* d_o, void* workspace, size_t workspace_bytes,
                         const qkmla_train_grads* grads, void* stream);

/*
 * Packed sequences of different lengths (prefill of a batch of prompts):
 * n_seqs sequences laid end to end over total_tokens token rows.  Every
 * [B][T]... array above becomes [total_tokens]...; sequence s holds rows
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 and its token i sits at position i.
 *   cu_seqlens   device int32 [n_seqs + 1]: 0 = cu[0] <= cu[1] <= ... <=
 *                cu[n_seqs] = total_tokens
 *   max_seq_len  host bound on every cu[s+1] - cu[s] (>= 1)
 *   status       device int32, nullable: QKMLA_DEV_BAD_SEQ_LEN if cu_seqlens
 *                breaks the rules above; every access stays in bounds, the
 *                outputs are then undefined
 * The fixed-length calls are these with cu_seqlens[s] = s * seq_len.  At most
 * 65535 sequences and 2^24 token rows per call (QKMLA_ERR_UNSUPPORTED).  o
 * must be 16-byte aligned.
 */
size_t qkmla_train_workspace_size_varlen(const qkmla_config* cfg, int32_t n_seqs,
                                         int32_t total_tokens, int32_t max_seq_len);
int qkmla_train_forward_varlen(const qkmla_config* cfg, int32_t n_seqs, const int32_t* cu_seqlens,
                               int32_t total_tokens, int32_t max_seq_len,
                               const qkmla_train_inputs* inputs, void* workspace,
                               size_t workspace_bytes, float* o, float* lse, int32_t* status,
                               void* stream);
int qkmla_train_backward_varlen(const qkmla_config* cfg, int32_t n_seqs,
                                const int32_t* cu_seqlens, int32_t total_tokens,
                                int32_t max_seq_len, const qkmla_train_inputs* inputs,
                                const float* o, const float* lse, const float* d_o,
                                void* workspace, size_t workspace_bytes,
                                const qkmla_train_grads* grads, int32_t* status, void* stream);

/*
 * Host-only split planner (no device access; usable without a GPU).  For a
 * decode of `batch` sequences bounded by max_seq_len on a device with n_cu
 * compute units, returns the number of decode workgroups and the token tile.
 */
int qkmla_plan(const qkmla_config* cfg, int32_t batch, int32_t max_seq_len, int32_t n_cu,
               int32_t* n_workgroups, int32_t* tile_tokens);

/*
 * Host-only plan inspection (no device access): the work split that
 * qkmla_decode's kernels use for these host-side sequence lengths and
 * n_workgroups (the value qkmla_plan returns).
 * qkmla_plan_segments writes one row of 5 int32 per segment into out[cap][5]:
 *   (workgroup, sequence, first tile, end tile (exclusive, tiles of the
 *    sequence), kind) with kind -1 = the segment is the whole sequence and is
 *   written as final output, 0/1 = partial written to that workgroup slot.
 * qkmla_plan_merge_sources writes the (workgroup, slot) pairs the merge reads
 * for sequence b into out[cap][2] (none if the sequence is written directly or
 * is invalid).  *n_out is the full count even when it exceeds cap.
 */
int qkmla_plan_segments(int32_t batch, const int32_t* seq_lens, int32_t cache_capacity,
                        int32_t n_workgroups, int32_t* out, int32_t cap, int32_t* n_out);
int qkmla_plan_merge_sources(int32_t batch, const int32_t* seq_lens, int32_t cache_capacity,
                             int32_t n_workgroups, int32_t b, int32_t* out, int32_t cap,
                             int32_t* n_out);

/*
 * Measurement hook.  Between qkmla_profile_begin() and qkmla_profile_end(),
 * every decode call (qkmla_decode, _multi, _paged, _noalloc) of this host
 * thread records HIP events on its stream before and after each of its
 * q-prep, split-KV and merge launches.  qkmla_profile_begin_reps(reps), reps
 * in 1..64, makes every decode call launch each of the three kernels reps
 * times back to back between its two events (each launch rewrites the same
 * outputs from the same inputs, so the call's results are unchanged) and
 * report the time per launch: the events' own latency, some microseconds,
 * is then spread over reps kernels.
 * qkmla_profile_end() waits for the recorded events and returns the summed
 * kernel time in milliseconds and the number of decode calls.  At most 4096
 * calls are recorded per begin/end window; the events are created on first
 * use and kept for the life of the process.  Not for use under stream
 * capture.
 */
int qkmla_profile_begin(void);
int qkmla_profile_begin_reps(int32_t reps);
int qkmla_profile_end(double* split_kv_ms_total, int32_t* launches);
/* The same window split by kernel: ms_total[0] q-prep, [1] the split-KV
 * kernel (the row-parallel decode for float storage), [2] the merge (0 for
 * float storage), summed over the recorded decode calls.  Ends the window
 * like qkmla_profile_end; use one of the two. */
int qkmla_profile_end_detail(double* ms_total, int32_t* launches);

const char* qkmla_status_string(int status);
const char* qkmla_last_error(void);
int qkmla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QKMLA_H_ */
