// Host side of the C ABI declared in include/qkmla.h: argument validation,
// the split planner, workspace layout and kernel dispatch.  Nothing here
// touches the GPU until a launcher is called, so validation errors and the
// planner can be exercised without a device.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <vector>

#include "plan_device.h"
#include "qkmla_internal.h"

namespace qkmla {
namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return QKMLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Validate the config and fill the normalised form.
// decode_shapes: apply the bf16 decode kernels' shape restrictions (the
// training kernels take any shape within their own limits).
int check_cfg(const qkmla_config* cfg, Cfg* out, bool decode_shapes = true) {
  if (!cfg) return fail(QKMLA_ERR_INVALID_ARG, "cfg is NULL");
  const qkmla_config& c = *cfg;
  if (c.n_heads <= 0 || c.n_groups <= 0 || c.latent_rank <= 0 || c.head_dim <= 0 ||
      c.rope_dim <= 0 || c.v_head_dim <= 0)
    return fail(QKMLA_ERR_INVALID_ARG, "all dimensions must be positive");
  if (c.n_heads % c.n_groups != 0)
    return fail(QKMLA_ERR_INVALID_ARG, "n_heads (%d) must be a multiple of n_groups (%d)",
                c.n_heads, c.n_groups);
  if (c.rope_dim % 2 != 0) return fail(QKMLA_ERR_INVALID_ARG, "rope_dim must be even");
  if (c.dtype != QKMLA_F32 && c.dtype != QKMLA_BF16)
    return fail(QKMLA_ERR_INVALID_ARG, "unknown dtype %d", c.dtype);
  if (c.qk_norm != 0 && c.qk_norm != 1) return fail(QKMLA_ERR_INVALID_ARG, "qk_norm must be 0 or 1");
  if (!(c.eps >= 0.f) || !std::isfinite(c.eps)) return fail(QKMLA_ERR_INVALID_ARG, "eps must be >= 0");
  if (!(c.rope_base > 0.f) || !std::isfinite(c.rope_base))
    return fail(QKMLA_ERR_INVALID_ARG, "rope_base must be > 0");
  if (!std::isfinite(c.softmax_scale)) return fail(QKMLA_ERR_INVALID_ARG, "softmax_scale not finite");
  if (c.latent_rank > 1024 || c.head_dim > 1024 || c.v_head_dim > 1024 || c.rope_dim > 256)
    return fail(QKMLA_ERR_UNSUPPORTED, "dimension above the compiled limits (r, d_c, d_v <= 1024, d_r <= 256)");
  if (c.dtype == QKMLA_BF16 && decode_shapes) {
    const int hpg = c.n_heads / c.n_groups;
    const bool h_ok = c.n_heads == 32 || c.n_heads == 64 || c.n_heads == 128;
    if (c.latent_rank != 512 || c.rope_dim != 64 || !h_ok || hpg != 16 || c.head_dim % 32 != 0 ||
        c.head_dim > 256)
      return fail(QKMLA_ERR_UNSUPPORTED,
                  "bf16 path is compiled for r=512, d_r=64, H in {32,64,128}, H/G=16, d_c in "
                  "{32,64,...,256} "
                  "(got r=%d d_r=%d H=%d G=%d d_c=%d)",
                  c.latent_rank, c.rope_dim, c.n_heads, c.n_groups, c.head_dim);
  }
  out->H = c.n_heads;
  out->G = c.n_groups;
  out->r = c.latent_rank;
  out->dc = c.head_dim;
  out->dr = c.rope_dim;
  out->dv = c.v_head_dim;
  out->dtype = c.dtype;
  out->qk_norm = c.qk_norm;
  out->eps = c.eps;
  out->tau = c.softmax_scale > 0.f ? c.softmax_scale
                                   : (float)(1.0 / std::sqrt((double)(c.head_dim + c.rope_dim)));
  out->base = c.rope_base;
  out->hpg = c.n_heads / c.n_groups;
  return QKMLA_OK;
}

size_t elem_size(const Cfg& c) { return c.dtype == QKMLA_BF16 ? 2 : 4; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

int plan_n_wg(const Cfg& c, int batch, int max_seq_len, int n_cu) {
  const int64_t tiles_bound = (int64_t)batch * ((max_seq_len + kTile - 1) / kTile);
  int forced = env_int("QKMLA_NUM_WG", 0);
  int64_t n = forced > 0 ? forced : n_cu;
  if (n > tiles_bound) n = tiles_bound;
  if (n < 1) n = 1;
  return (int)n;
}

// Compute units of the current device, queried once per device and kept, so
// that a decode call recorded into a HIP graph makes no attribute query.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0)
    return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Measurement hook state (per host thread): per recorded decode call, HIP
// events on its stream before and after each of its three kernels (q-prep 0,
// split-KV 1, merge 2).  With reps > 1 each kernel is launched reps times back
// to back between its two events (every launch rewrites the same outputs from
// the same inputs), so that the events' own latency is spread over reps
// kernels.  A path without a merge records that pair back to back.
constexpr int kTimedMax = 4096;
struct KernelTimer {
  bool on = false;
  int reps = 1;
  int n = 0;
  hipEvent_t ev[3][2][kTimedMax];
  int created = 0;
};
thread_local KernelTimer g_timer;

hipError_t timer_record(hipStream_t s, int which, int edge) {
  KernelTimer& t = g_timer;
  if (t.n >= t.created) {
    for (int k = 0; k < 3; ++k)
      for (int j = 0; j < 2; ++j) {
        const hipError_t e = hipEventCreate(&t.ev[k][j][t.n]);
        if (e != hipSuccess) return e;
      }
    t.created = t.n + 1;
  }
  return hipEventRecord(t.ev[which][edge][t.n], s);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QKMLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

WsLayout ws_layout(const Cfg& c, int batch, int n_wg) {
  WsLayout w;
  const size_t es = elem_size(c);
  size_t off = 0;
  w.q_tilde = off;
  off = align256(off + (size_t)batch * c.H * c.r * es);
  w.alpha_q = off;
  off = align256(off + (size_t)batch * c.H * 4);
  w.q_rope = off;
  off = align256(off + (size_t)batch * c.H * c.dr * es);
  w.partials = off;
  if (c.dtype == QKMLA_BF16) off = align256(off + (size_t)n_wg * kSlotsPerWg * kPartialSlotBytes(c.H, c.r));
  w.plan = off;
  if (c.dtype == QKMLA_BF16) off = align256(off + (size_t)(batch + 1) * 4);
  w.total = off;
  return w;
}

}  // namespace qkmla

using namespace qkmla;

extern "C" {

int qkmla_abi_version(void) { return QKMLA_ABI_VERSION; }

int qkmla_profile_begin(void) { return qkmla_profile_begin_reps(1); }

int qkmla_profile_begin_reps(int32_t reps) {
  if (reps < 1 || reps > 64) return fail(QKMLA_ERR_INVALID_ARG, "profile: reps must be in 1..64");
  g_timer.on = true;
  g_timer.reps = reps;
  g_timer.n = 0;
  return ok();
}

int qkmla_profile_end_detail(double* ms_total, int32_t* launches) {
  KernelTimer& t = g_timer;
  t.on = false;
  double total[3] = {0.0, 0.0, 0.0};
  for (int i = 0; i < t.n; ++i) {
    hipError_t e = hipEventSynchronize(t.ev[2][1][i]);
    for (int k = 0; k < 3 && e == hipSuccess; ++k) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, t.ev[k][0][i], t.ev[k][1][i]);
      total[k] += ms / t.reps;
    }
    if (e != hipSuccess) return hip_status(e, "profile_end");
  }
  if (ms_total)
    for (int k = 0; k < 3; ++k) ms_total[k] = total[k];
  if (launches) *launches = t.n;
  t.n = 0;
  return ok();
}

int qkmla_profile_end(double* split_kv_ms_total, int32_t* launches) {
  double ms[3];
  const int st = qkmla_profile_end_detail(ms, launches);
  if (st) return st;
  if (split_kv_ms_total) *split_kv_ms_total = ms[1];
  return ok();
}

const char* qkmla_last_error(void) { return g_err; }

const char* qkmla_status_string(int status) {
  switch (status) {
    case QKMLA_OK: return "ok";
    case QKMLA_ERR_INVALID_ARG: return "invalid argument";
    case QKMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case QKMLA_ERR_WORKSPACE: return "workspace too small";
    case QKMLA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int qkmla_plan(const qkmla_config* cfg, int32_t batch, int32_t max_seq_len, int32_t n_cu,
               int32_t* n_workgroups, int32_t* tile_tokens) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || max_seq_len < 1 || n_cu < 1 || !n_workgroups || !tile_tokens)
    return fail(QKMLA_ERR_INVALID_ARG, "bad plan arguments");
  *tile_tokens = kTile;
  *n_workgroups = batch == 0 ? 0 : plan_n_wg(c, batch, max_seq_len, n_cu);
  return ok();
}

// Host replay of the decode plan (same helpers as the kernels).
static int host_prefix(int32_t batch, const int32_t* seq_lens, int32_t L_cap, std::vector<int>* P) {
  if (batch < 0 || batch > kMaxBatch || (batch > 0 && !seq_lens) || L_cap < 1)
    return fail(QKMLA_ERR_INVALID_ARG, "plan: bad batch, lengths or capacity");
  P->assign(batch + 1, 0);
  for (int b = 0; b < batch; ++b) (*P)[b + 1] = (*P)[b] + tiles_of(seq_lens[b], L_cap);
  return QKMLA_OK;
}

int qkmla_plan_segments(int32_t batch, const int32_t* seq_lens, int32_t cache_capacity,
                        int32_t n_wg, int32_t* out, int32_t cap, int32_t* n_out) {
  std::vector<int> P;
  int st = host_prefix(batch, seq_lens, cache_capacity, &P);
  if (st) return st;
  if (n_wg < 1 || !n_out || (cap > 0 && !out)) return fail(QKMLA_ERR_INVALID_ARG, "plan: bad output");
  const int64_t N = P[batch];
  int n = 0;
  for (int p = 0; p < n_wg && N > 0; ++p) {
    int64_t x = wg_start(p, N, n_wg);
    const int64_t e = wg_start(p + 1, N, n_wg);
    bool first = true;
    while (x < e) {  // the decode kernel's segment loop
      const int b = seq_of(P.data(), batch, x);
      const int64_t s0 = P[b], s1 = P[b + 1];
      const int64_t seg_end = e < s1 ? e : s1;
      const bool complete = (x == s0) && (seg_end == s1);
      if (n < cap) {
        int32_t* r = out + 5 * n;
        r[0] = p;
        r[1] = b;
        r[2] = (int32_t)(x - s0);
        r[3] = (int32_t)(seg_end - s0);
        r[4] = complete ? -1 : (first ? 0 : 1);
      }
      ++n;
      first = false;
      x = seg_end;
    }
  }
  *n_out = n;
  return ok();
}

int qkmla_plan_merge_sources(int32_t batch, const int32_t* seq_lens, int32_t cache_capacity,
                             int32_t n_wg, int32_t b, int32_t* out, int32_t cap, int32_t* n_out) {
  std::vector<int> P;
  int st = host_prefix(batch, seq_lens, cache_capacity, &P);
  if (st) return st;
  if (n_wg < 1 || b < 0 || b >= batch || !n_out || (cap > 0 && !out))
    return fail(QKMLA_ERR_INVALID_ARG, "plan: bad merge query");
  const int64_t N = P[batch];
  int n = 0;
  if (P[b + 1] > P[b]) {
    const int p_lo = wg_of(P[b], N, n_wg), p_hi = wg_of(P[b + 1] - 1, N, n_wg);
    if (p_lo != p_hi) {  // the merge kernel's source loop
      for (int p = p_lo; p <= p_hi; ++p) {
        const int slot = merge_slot(P.data(), b, N, n_wg, p);
        if (slot < 0) continue;
        if (n < cap) {
          out[2 * n] = p;
          out[2 * n + 1] = slot;
        }
        ++n;
      }
    }
  }
  *n_out = n;
  return ok();
}

int qkmla_absorb_weights(const qkmla_config* cfg, const float* w_uk, const float* gamma_q,
                         const float* gamma_k, void* w_qabs, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (!w_uk || !w_qabs || (c.qk_norm && (!gamma_q || !gamma_k)))
    return fail(QKMLA_ERR_INVALID_ARG, "absorb: NULL pointer");
  if (!aligned(w_uk, 4) || !aligned(w_qabs, elem_size(c)))
    return fail(QKMLA_ERR_INVALID_ARG, "absorb: pointers must be aligned to their element size");
  return hip_status(launch_absorb(c, w_uk, gamma_q, gamma_k, w_qabs, as_stream(stream)), "absorb");
}

// Checks a caller's page description; on success *pg describes it.
static int check_pages(const qkmla_pages* pages, const char* who, Paging* pg) {
  if (!pages || !pages->block_table)
    return fail(QKMLA_ERR_INVALID_ARG, "%s: NULL page description or block table", who);
  if (pages->max_blocks < 1 || pages->page_size < 1 || pages->num_pages < 1)
    return fail(QKMLA_ERR_INVALID_ARG, "%s: max_blocks, page_size and num_pages must be >= 1", who);
  if ((int64_t)pages->max_blocks * pages->page_size > INT32_MAX)
    return fail(QKMLA_ERR_INVALID_ARG, "%s: max_blocks * page_size above 2^31 - 1", who);
  if (!aligned(pages->block_table, 4))
    return fail(QKMLA_ERR_INVALID_ARG, "%s: block table must be 4-byte aligned", who);
  *pg = Paging{pages->block_table, pages->max_blocks, pages->page_size, pages->num_pages};
  return QKMLA_OK;
}

static int append_impl(const Cfg& c, int32_t batch, int32_t n_new, const void* c_new,
                       const void* k_rope_new, const float* w_uk, const float* gamma_k_rope,
                       const int32_t* positions, const Paging& pg, void* latent_cache,
                       void* rope_cache, float* alpha_cache, int32_t* status, void* stream) {
  if ((int64_t)batch * n_new > (int64_t)1 << 30)
    return fail(QKMLA_ERR_UNSUPPORTED, "append: too many tokens in one call");
  if (!c_new || !k_rope_new || !positions || !latent_cache || !rope_cache ||
      (c.qk_norm && (!w_uk || !gamma_k_rope || !alpha_cache)))
    return fail(QKMLA_ERR_INVALID_ARG, "append: NULL pointer");
  const size_t es = elem_size(c);
  if (!aligned(c_new, es) || !aligned(k_rope_new, es) || !aligned(latent_cache, es) ||
      !aligned(rope_cache, es) || (alpha_cache && !aligned(alpha_cache, 4)) ||
      (w_uk && !aligned(w_uk, 4)) || !aligned(positions, 4))
    return fail(QKMLA_ERR_INVALID_ARG, "append: pointers must be aligned to their element size");
  return hip_status(launch_append(c, batch, n_new, c_new, k_rope_new, w_uk, gamma_k_rope, positions,
                                  pg, latent_cache, rope_cache, alpha_cache, status,
                                  as_stream(stream)),
                    "append");
}

int qkmla_append(const qkmla_config* cfg, int32_t batch, int32_t n_new, const void* c_new,
                 const void* k_rope_new, const float* w_uk, const float* gamma_k_rope,
                 const int32_t* positions, int32_t cache_capacity, void* latent_cache,
                 void* rope_cache, float* alpha_cache, int32_t* status, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || n_new < 0 || cache_capacity < 1)
    return fail(QKMLA_ERR_INVALID_ARG, "append: batch/n_new must be >= 0, cache_capacity >= 1");
  if (batch == 0 || n_new == 0) return ok();
  return append_impl(c, batch, n_new, c_new, k_rope_new, w_uk, gamma_k_rope, positions,
                     contiguous_paging(batch, cache_capacity), latent_cache, rope_cache,
                     alpha_cache, status, stream);
}

int qkmla_append_paged(const qkmla_config* cfg, int32_t batch, int32_t n_new, const void* c_new,
                       const void* k_rope_new, const float* w_uk, const float* gamma_k_rope,
                       const int32_t* positions, const qkmla_pages* pages, void* latent_pool,
                       void* rope_pool, float* alpha_pool, int32_t* status, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || n_new < 0)
    return fail(QKMLA_ERR_INVALID_ARG, "append: batch/n_new must be >= 0");
  if (batch == 0 || n_new == 0) return ok();
  Paging pg;
  if ((st = check_pages(pages, "append", &pg))) return st;
  return append_impl(c, batch, n_new, c_new, k_rope_new, w_uk, gamma_k_rope, positions, pg,
                     latent_pool, rope_pool, alpha_pool, status, stream);
}

size_t qkmla_decode_workspace_size(const qkmla_config* cfg, int32_t batch, int32_t max_seq_len) {
  Cfg c;
  if (check_cfg(cfg, &c)) return 0;
  if (batch < 0 || max_seq_len < 1) {
    fail(QKMLA_ERR_INVALID_ARG, "workspace size: batch >= 0 and max_seq_len >= 1 required");
    return 0;
  }
  if (batch == 0) return 256;
  const int n_wg = plan_n_wg(c, batch, max_seq_len, device_cu_count());
  return ws_layout(c, batch, n_wg).total;
}

static int decode_impl(const Cfg& c, int32_t batch, int32_t s_q, const void* q_c,
                       const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                       const void* latent_cache, const void* rope_cache, const float* alpha_cache,
                       const int32_t* seq_lens, const Paging& pg, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                       int32_t* status, void* stream) {
  if ((int64_t)batch * s_q > kMaxBatch)
    return fail(QKMLA_ERR_UNSUPPORTED, "decode: batch * s_q above %d", kMaxBatch);
  if (!q_c || !q_rope || !w_qabs || !latent_cache || !rope_cache || !seq_lens || !workspace ||
      !o_lat || (c.qk_norm && (!gamma_q_rope || !alpha_cache)))
    return fail(QKMLA_ERR_INVALID_ARG, "decode: NULL pointer");
  // The bf16 path reads queries, weights and cache rows as 16-byte vectors.
  const size_t va = c.dtype == QKMLA_BF16 ? 16 : 4;
  if (!aligned(q_c, va) || !aligned(q_rope, va) || !aligned(w_qabs, va) ||
      !aligned(latent_cache, va) || !aligned(rope_cache, va) ||
      (alpha_cache && !aligned(alpha_cache, 4)) || !aligned16(workspace) || !aligned(o_lat, va) ||
      (lse && !aligned(lse, 4)) || !aligned(seq_lens, 4))
    return fail(QKMLA_ERR_INVALID_ARG,
                "decode: pointers must be %zu-byte aligned (alpha, lse, seq_lens: 4; workspace: 16)", va);
  // The split-KV kernel loads whole 32-row tiles from one page.
  if (c.dtype == QKMLA_BF16 && pg.bt && pg.page_size % kTile != 0)
    return fail(QKMLA_ERR_UNSUPPORTED, "decode: bf16 pages must hold a multiple of %d rows", kTile);
  hipStream_t s = as_stream(stream);
  const int nv = batch * s_q;  // one virtual sequence per query row
  const int n_wg = plan_n_wg(c, nv, max_seq_len, device_cu_count());
  const WsLayout ws = ws_layout(c, nv, n_wg);
  if (workspace_bytes < ws.total)
    return fail(QKMLA_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu", workspace_bytes,
                ws.total);
  const bool timed = g_timer.on && g_timer.n < kTimedMax;
  const int reps = timed ? g_timer.reps : 1;
  hipError_t e = hipSuccess;
  if (timed && (e = timer_record(s, 0, 0)) != hipSuccess) return hip_status(e, "decode/timer");
  for (int i = 0; i < reps && e == hipSuccess; ++i)
    e = launch_qprep(c, batch, s_q, q_c, q_rope, w_qabs, gamma_q_rope, seq_lens, pg, ws, workspace,
                     status, s);
  if (e != hipSuccess) return hip_status(e, "decode/qprep");
  if (timed && ((e = timer_record(s, 0, 1)) != hipSuccess || (e = timer_record(s, 1, 0)) != hipSuccess))
    return hip_status(e, "decode/timer");
  if (c.dtype == QKMLA_BF16) {
    for (int i = 0; i < reps && e == hipSuccess; ++i)
      e = launch_decode_mfma(c, batch, s_q, seq_lens, pg, latent_cache, rope_cache, alpha_cache, ws,
                             workspace, n_wg, o_lat, lse, s);
    if (e != hipSuccess) return hip_status(e, "decode/splitkv");
    if (timed && ((e = timer_record(s, 1, 1)) != hipSuccess || (e = timer_record(s, 2, 0)) != hipSuccess))
      return hip_status(e, "decode/timer");
    for (int i = 0; i < reps && e == hipSuccess; ++i)
      e = launch_merge(c, batch, s_q, ws, workspace, n_wg, o_lat, lse, s);
    if (e != hipSuccess) return hip_status(e, "decode/merge");
  } else {
    for (int i = 0; i < reps && e == hipSuccess; ++i)
      e = launch_decode_generic(c, batch, s_q, seq_lens, pg, latent_cache, rope_cache, alpha_cache,
                                ws, workspace, o_lat, lse, s);
    if (e != hipSuccess) return hip_status(e, "decode/generic");
    if (timed && ((e = timer_record(s, 1, 1)) != hipSuccess || (e = timer_record(s, 2, 0)) != hipSuccess))
      return hip_status(e, "decode/timer");
  }
  if (timed) {
    if ((e = timer_record(s, 2, 1)) != hipSuccess) return hip_status(e, "decode/timer");
    ++g_timer.n;
  }
  return ok();
}

int qkmla_decode_multi(const qkmla_config* cfg, int32_t batch, int32_t s_q, const void* q_c,
                       const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                       const void* latent_cache, const void* rope_cache, const float* alpha_cache,
                       const int32_t* seq_lens, int32_t cache_capacity, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                       int32_t* status, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || s_q < 1 || cache_capacity < 1 || max_seq_len < 1 ||
      max_seq_len > cache_capacity)
    return fail(QKMLA_ERR_INVALID_ARG,
                "decode: need batch >= 0, s_q >= 1 and 1 <= max_seq_len (%d) <= cache_capacity (%d)",
                max_seq_len, cache_capacity);
  if (batch == 0) return ok();
  return decode_impl(c, batch, s_q, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache, rope_cache,
                     alpha_cache, seq_lens, contiguous_paging(batch, cache_capacity), max_seq_len,
                     workspace, workspace_bytes, o_lat, lse, status, stream);
}

int qkmla_decode_paged(const qkmla_config* cfg, int32_t batch, int32_t s_q, const void* q_c,
                       const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                       const void* latent_pool, const void* rope_pool, const float* alpha_pool,
                       const int32_t* seq_lens, const qkmla_pages* pages, int32_t max_seq_len,
                       void* workspace, size_t workspace_bytes, float* o_lat, float* lse,
                       int32_t* status, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || s_q < 1 || max_seq_len < 1)
    return fail(QKMLA_ERR_INVALID_ARG, "decode: need batch >= 0, s_q >= 1, max_seq_len >= 1");
  if (batch == 0) return ok();
  Paging pg;
  if ((st = check_pages(pages, "decode", &pg))) return st;
  if (max_seq_len > pg.capacity())
    return fail(QKMLA_ERR_INVALID_ARG, "decode: max_seq_len (%d) above max_blocks * page_size (%d)",
                max_seq_len, pg.capacity());
  return decode_impl(c, batch, s_q, q_c, q_rope, w_qabs, gamma_q_rope, latent_pool, rope_pool,
                     alpha_pool, seq_lens, pg, max_seq_len, workspace, workspace_bytes, o_lat, lse,
                     status, stream);
}

int qkmla_decode(const qkmla_config* cfg, int32_t batch, const void* q_c, const void* q_rope,
                 const void* w_qabs, const float* gamma_q_rope, const void* latent_cache,
                 const void* rope_cache, const float* alpha_cache, const int32_t* seq_lens,
                 int32_t cache_capacity, int32_t max_seq_len, void* workspace,
                 size_t workspace_bytes, float* o_lat, float* lse, int32_t* status,
                 void* stream) {
  return qkmla_decode_multi(cfg, batch, 1, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache,
                            rope_cache, alpha_cache, seq_lens, cache_capacity, max_seq_len,
                            workspace, workspace_bytes, o_lat, lse, status, stream);
}

// ---- decode without a caller workspace ------------------------------------------------
// The workspace of qkmla_decode_noalloc: one array per GPU, placed by the code
// object loader and held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol); each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is what the kernels receive.
static __device__ __align__(256) char scratch[QKMLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// This device's address of `scratch`, or nullptr with the error recorded.
void* scratch_address(int* st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, "decode_noalloc/hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    *st = fail(QKMLA_ERR_UNSUPPORTED, "decode_noalloc: device %d beyond the %d the library serves",
               dev, kMaxScratchDevices);
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *st = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "decode_noalloc/hipGetSymbolAddress");
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}
}  // namespace

int qkmla_decode_noalloc(const qkmla_config* cfg, int32_t batch, const void* q_c,
                         const void* q_rope, const void* w_qabs, const float* gamma_q_rope,
                         const void* latent_cache, const void* rope_cache,
                         const float* alpha_cache, const int32_t* seq_lens,
                         int32_t cache_capacity, int32_t max_seq_len, float* o_lat, float* lse,
                         int32_t* status, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0 || cache_capacity < 1 || max_seq_len < 1 || max_seq_len > cache_capacity)
    return fail(QKMLA_ERR_INVALID_ARG,
                "decode_noalloc: need batch >= 0 and 1 <= max_seq_len (%d) <= cache_capacity (%d)",
                max_seq_len, cache_capacity);
  if (batch == 0) return ok();
  if (batch > kMaxBatch)
    return fail(QKMLA_ERR_UNSUPPORTED, "decode_noalloc: batch above %d", kMaxBatch);
  const size_t need = qkmla_decode_workspace_size(cfg, batch, max_seq_len);
  if (need == 0) return QKMLA_ERR_INVALID_ARG;  // message set by the size query
  if (need > (size_t)QKMLA_NOALLOC_SCRATCH_BYTES)
    return fail(QKMLA_ERR_WORKSPACE,
                "decode_noalloc: this batch needs %zu bytes of workspace, above the %zu-byte "
                "scratch array; use qkmla_decode with a caller workspace",
                need, (size_t)QKMLA_NOALLOC_SCRATCH_BYTES);
  void* ws = scratch_address(&st);
  if (!ws) return st;
  return decode_impl(c, batch, 1, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache, rope_cache,
                     alpha_cache, seq_lens, contiguous_paging(batch, cache_capacity), max_seq_len,
                     ws, (size_t)QKMLA_NOALLOC_SCRATCH_BYTES, o_lat, lse, status, stream);
}

// ---- training / prefill -------------------------------------------------------------
// Packed form: n_seq sequences over n_rows rows, each at most max_len long.
static int check_train(const qkmla_config* cfg, int64_t n_seq, int64_t n_rows, int64_t max_len,
                       Cfg* c) {
  int st = check_cfg(cfg, c, false);
  if (st) return st;
  if (n_seq < 0 || n_rows < 0 || max_len < 1)
    return fail(QKMLA_ERR_INVALID_ARG, "train: need sequences >= 0, tokens >= 0, max length >= 1");
  if (c->dc > 256 || c->dv > 256)
    return fail(QKMLA_ERR_UNSUPPORTED, "train: d_c and d_v must be <= 256 (got %d, %d)", c->dc,
                c->dv);
  // row-per-block kernels launch n_rows blocks of 256 threads; the dispatch
  // size in work-items must fit 32 bits
  if (n_rows * c->H > INT32_MAX / 2 || max_len > INT32_MAX / 2 || n_rows > (1 << 24))
    return fail(QKMLA_ERR_UNSUPPORTED, "train: more than 2^24 tokens or tokens * n_heads too large");
  if (n_seq > 65535) return fail(QKMLA_ERR_UNSUPPORTED, "train: more than 65535 sequences");
  return QKMLA_OK;
}

static int check_train_inputs(const Cfg& c, const qkmla_train_inputs* in, TrainPtrs* p) {
  if (!in) return fail(QKMLA_ERR_INVALID_ARG, "train: NULL inputs");
  if (!in->c || !in->q_c || !in->q_rope || !in->k_rope || !in->w_uk || !in->w_uv ||
      (c.qk_norm && (!in->gamma_q || !in->gamma_k || !in->gamma_q_rope || !in->gamma_k_rope)))
    return fail(QKMLA_ERR_INVALID_ARG, "train: NULL input pointer");
  const size_t es = elem_size(c);
  if (!aligned(in->c, es) || !aligned(in->q_c, es) || !aligned(in->q_rope, es) ||
      !aligned(in->k_rope, es) || !aligned(in->w_uv, es) || !aligned(in->w_uk, 4))
    return fail(QKMLA_ERR_INVALID_ARG, "train: inputs must be aligned to their element size");
  // the MFMA path reads latents, W^UV and the bf16 operands as 16-byte vectors
  if (train_mfma_shape(c) && (!aligned(in->c, 16) || !aligned(in->w_uv, 16)))
    return fail(QKMLA_ERR_INVALID_ARG, "train: bf16 latents and W^UV must be 16-byte aligned");
  *p = TrainPtrs{in->c, in->q_c, in->q_rope, in->k_rope, in->w_uk, in->w_uv,
                 in->gamma_q, in->gamma_k, in->gamma_q_rope, in->gamma_k_rope};
  return QKMLA_OK;
}

static int train_forward(const Cfg& c, const TrainSeqs& q, const qkmla_train_inputs* inputs,
                         void* workspace, size_t workspace_bytes, float* o, float* lse,
                         int32_t* status, void* stream) {
  TrainPtrs in;
  int st = check_train_inputs(c, inputs, &in);
  if (st) return st;
  if (!workspace || !o || !lse) return fail(QKMLA_ERR_INVALID_ARG, "train: NULL pointer");
  if (!aligned16(workspace) || !aligned(o, 16) || !aligned(lse, 4) || (status && !aligned(status, 4)))
    return fail(QKMLA_ERR_INVALID_ARG, "train: misaligned workspace or output (o: 16 bytes)");
  const TrainWs ws = train_ws_layout(c, q);
  if (workspace_bytes < ws.fwd_total)
    return fail(QKMLA_ERR_WORKSPACE, "train forward: workspace %zu bytes, need %zu",
                workspace_bytes, ws.fwd_total);
  return hip_status(
      launch_train_forward(c, q, in, ws, workspace, o, lse, status, as_stream(stream)),
      "train forward");
}

static int train_backward(const Cfg& c, const TrainSeqs& q, const qkmla_train_inputs* inputs,
                          const float* o, const float* lse, const float* d_o, void* workspace,
                          size_t workspace_bytes, const qkmla_train_grads* grads, int32_t* status,
                          void* stream) {
  TrainPtrs in;
  int st = check_train_inputs(c, inputs, &in);
  if (st) return st;
  if (!o || !lse || !d_o || !workspace || !grads)
    return fail(QKMLA_ERR_INVALID_ARG, "train: NULL pointer");
  const qkmla_train_grads& g = *grads;
  float* outs[] = {g.d_c, g.d_q_c, g.d_q_rope, g.d_k_rope, g.d_w_uk, g.d_w_uv,
                   g.d_gamma_q, g.d_gamma_k, g.d_gamma_q_rope, g.d_gamma_k_rope};
  for (float* p : outs)
    if (!p || !aligned(p, 4)) return fail(QKMLA_ERR_INVALID_ARG, "train: NULL or misaligned gradient");
  if (!aligned16(workspace) || !aligned(o, 8) || !aligned(lse, 4) || !aligned(d_o, 8) ||
      (status && !aligned(status, 4)))
    return fail(QKMLA_ERR_INVALID_ARG, "train: misaligned workspace, o, lse or d_o");
  const TrainWs ws = train_ws_layout(c, q);
  if (workspace_bytes < ws.total)
    return fail(QKMLA_ERR_WORKSPACE, "train backward: workspace %zu bytes, need %zu",
                workspace_bytes, ws.total);
  const TrainGrads gr{g.d_c, g.d_q_c, g.d_q_rope, g.d_k_rope, g.d_w_uk, g.d_w_uv,
                      g.d_gamma_q, g.d_gamma_k, g.d_gamma_q_rope, g.d_gamma_k_rope};
  return hip_status(launch_train_backward(c, q, in, o, lse, d_o, ws, workspace, gr, status,
                                          as_stream(stream)),
                    "train backward");
}

size_t qkmla_train_workspace_size(const qkmla_config* cfg, int32_t batch, int32_t seq_len) {
  Cfg c;
  if (check_train(cfg, batch, (int64_t)batch * seq_len, seq_len, &c)) return 0;
  if (batch == 0) return 256;
  return train_ws_layout(c, TrainSeqs{batch * seq_len, batch, seq_len, nullptr}).total;
}

int qkmla_train_forward(const qkmla_config* cfg, int32_t batch, int32_t seq_len,
                        const qkmla_train_inputs* inputs, void* workspace, size_t workspace_bytes,
                        float* o, float* lse, void* stream) {
  Cfg c;
  int st = check_train(cfg, batch, (int64_t)batch * seq_len, seq_len, &c);
  if (st) return st;
  if (batch == 0) return ok();
  return train_forward(c, TrainSeqs{batch * seq_len, batch, seq_len, nullptr}, inputs, workspace,
                       workspace_bytes, o, lse, nullptr, stream);
}

int qkmla_train_backward(const qkmla_config* cfg, int32_t batch, int32_t seq_len,
                         const qkmla_train_inputs* inputs, const float* o, const float* lse,
                         const float* d_o, void* workspace, size_t workspace_bytes,
                         const qkmla_train_grads* grads, void* stream) {
  Cfg c;
  int st = check_train(cfg, batch, (int64_t)batch * seq_len, seq_len, &c);
  if (st) return st;
  if (batch == 0) return ok();
  return train_backward(c, TrainSeqs{batch * seq_len, batch, seq_len, nullptr}, inputs, o, lse,
                        d_o, workspace, workspace_bytes, grads, nullptr, stream);
}

size_t qkmla_train_workspace_size_varlen(const qkmla_config* cfg, int32_t n_seqs,
                                         int32_t total_tokens, int32_t max_seq_len) {
  Cfg c;
  if (check_train(cfg, n_seqs, total_tokens, max_seq_len, &c)) return 0;
  if (n_seqs == 0 || total_tokens == 0) return 256;
  return train_ws_layout(c, TrainSeqs{total_tokens, n_seqs, max_seq_len, nullptr}).total;
}

static int check_cu(const int32_t* cu_seqlens) {
  if (!cu_seqlens || !aligned(cu_seqlens, 4))
    return fail(QKMLA_ERR_INVALID_ARG, "train: cu_seqlens NULL or misaligned");
  return QKMLA_OK;
}

int qkmla_train_forward_varlen(const qkmla_config* cfg, int32_t n_seqs, const int32_t* cu_seqlens,
                               int32_t total_tokens, int32_t max_seq_len,
                               const qkmla_train_inputs* inputs, void* workspace,
                               size_t workspace_bytes, float* o, float* lse, int32_t* status,
                               void* stream) {
  Cfg c;
  int st = check_train(cfg, n_seqs, total_tokens, max_seq_len, &c);
  if (st) return st;
  if (n_seqs == 0 || total_tokens == 0) return ok();
  if ((st = check_cu(cu_seqlens))) return st;
  return train_forward(c, TrainSeqs{total_tokens, n_seqs, max_seq_len, cu_seqlens}, inputs,
                       workspace, workspace_bytes, o, lse, status, stream);
}

int qkmla_train_backward_varlen(const qkmla_config* cfg, int32_t n_seqs,
                                const int32_t* cu_seqlens, int32_t total_tokens,
                                int32_t max_seq_len, const qkmla_train_inputs* inputs,
                                const float* o, const float* lse, const float* d_o,
                                void* workspace, size_t workspace_bytes,
                                const qkmla_train_grads* grads, int32_t* status, void* stream) {
  Cfg c;
  int st = check_train(cfg, n_seqs, total_tokens, max_seq_len, &c);
  if (st) return st;
  if (n_seqs == 0 || total_tokens == 0) return ok();
  if ((st = check_cu(cu_seqlens))) return st;
  return train_backward(c, TrainSeqs{total_tokens, n_seqs, max_seq_len, cu_seqlens}, inputs, o,
                        lse, d_o, workspace, workspace_bytes, grads, status, stream);
}

int qkmla_out_proj(const qkmla_config* cfg, int32_t batch, const float* o_lat, const void* w_uv,
                   float* out, void* stream) {
  Cfg c;
  int st = check_cfg(cfg, &c);
  if (st) return st;
  if (batch < 0) return fail(QKMLA_ERR_INVALID_ARG, "out_proj: batch must be >= 0");
  if (batch == 0) return ok();
  if (!o_lat || !w_uv || !out) return fail(QKMLA_ERR_INVALID_ARG, "out_proj: NULL pointer");
  if (!aligned(o_lat, 4) || !aligned(w_uv, elem_size(c)) || !aligned(out, 4))
    return fail(QKMLA_ERR_INVALID_ARG, "out_proj: pointers must be aligned to their element size");
  if (out_proj_uses_mfma(c) && (!aligned(o_lat, 16) || !aligned(w_uv, 16)))
    return fail(QKMLA_ERR_INVALID_ARG, "out_proj: o_lat and w_uv must be 16-byte aligned");
  return hip_status(launch_out_proj(c, batch, o_lat, w_uv, out, as_stream(stream)), "out_proj");
}

}  // extern "C"
