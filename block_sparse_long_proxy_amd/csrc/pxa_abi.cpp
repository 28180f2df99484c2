// pxa_abi.cpp -- the extern "C" boundary (include/pxa.h): host-side
// validation, workspace layout and the launch sequence.  No allocation, no
// synchronisation, no global mutable state except a thread-local copy of the
// last HIP error message.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <utility>

#include "../../include/pxa.h"
#include "pxa_launch.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

constexpr int kMaxSeq = 524288;
constexpr int kMaxHeads = 1024;

int check_config(const pxa_config* c) {
  if (!c) return PXA_ENULL;
  if (c->num_heads < 1 || c->num_kv_heads < 1 || c->num_proxies < 1 || c->seq_len < 1)
    return PXA_EINVAL;
  if (c->num_heads > kMaxHeads || c->num_kv_heads > c->num_heads) return PXA_EINVAL;
  if (c->num_heads % c->num_kv_heads) return PXA_EINVAL;
  if (c->num_heads % c->num_proxies) return PXA_EINVAL;
  if ((c->num_kv_heads % c->num_proxies) && (c->num_proxies % c->num_kv_heads)) return PXA_EINVAL;
  if (!std::isfinite(c->gamma) || !(c->gamma > 0.f) || c->gamma > 1.f) return PXA_EINVAL;
  if (std::isnan(c->softmax_scale) || std::isinf(c->softmax_scale)) return PXA_EINVAL;
  if (c->block != pxa::kBlockTokens) return PXA_EUNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PXA_EUNSUPPORTED;
  if (c->seq_len > kMaxSeq) return PXA_EUNSUPPORTED;
  const int64_t nb = pxa::num_blocks(c->seq_len);   // the last block may be partial
  if ((int64_t)c->num_heads * nb * (nb + 1) / 2 > INT32_MAX) return PXA_EUNSUPPORTED;
  return PXA_OK;
}

// Method-variant check against a valid configuration; NULL is the default.
int check_budget(const pxa_config* c, const pxa_options* b) {
  if (!b) return PXA_OK;
  const int nb = pxa::num_blocks(c->seq_len);
  if (b->score_stride != 1 && b->score_stride != 2 && b->score_stride != 4) return PXA_EINVAL;
  if (!std::isfinite(b->skip_threshold) || b->skip_threshold < 0.f || b->skip_threshold > 1.f)
    return PXA_EINVAL;
  switch (b->budget_mode) {
    case PXA_BUDGET_DYNAMIC:
      if (b->last_blocks < 1 || b->last_blocks > nb || b->last_blocks > PXA_MAX_PROBE_BLOCKS)
        return PXA_EINVAL;
      return PXA_OK;
    case PXA_BUDGET_FIXED:
      return b->fixed_blocks >= 1 ? PXA_OK : PXA_EINVAL;
    case PXA_BUDGET_RATIO:
      return (std::isfinite(b->ratio) && b->ratio > 0.f && b->ratio <= 1.f) ? PXA_OK : PXA_EINVAL;
    default:
      return PXA_EINVAL;
  }
}

int check_all(const pxa_config* c, const pxa_options* b) {
  const int rc = check_config(c);
  return rc != PXA_OK ? rc : check_budget(c, b);
}

pxa::LaunchArgs args_of(const pxa_config* c, const pxa_options* b = nullptr) {
  pxa::LaunchArgs a;
  a.H = c->num_heads;
  a.Hkv = c->num_kv_heads;
  a.N = c->seq_len;
  a.D = c->head_dim;
  a.G = c->num_proxies;
  a.scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  a.gamma = c->gamma;
  if (b) {
    a.budget_mode = b->budget_mode;
    a.last_blocks = b->budget_mode == PXA_BUDGET_DYNAMIC ? b->last_blocks : 1;
    a.fixed_blocks = b->fixed_blocks;
    a.ratio = b->ratio;
    a.score_stride = b->score_stride;
    a.skip_threshold = b->skip_threshold;
  }
  return a;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int ptr_ok(const void* p, size_t a) {
  if (!p) return PXA_ENULL;
  if (!aligned(p, a)) return PXA_EALIGN;
  return PXA_OK;
}

// First non-OK code among the pointer checks.
int ptrs_ok(std::initializer_list<std::pair<const void*, size_t>> ps) {
  int rc = PXA_OK;
  for (auto& p : ps) {   // NULL is reported before misalignment
    const int r = ptr_ok(p.first, p.second);
    if (r == PXA_ENULL) return r;
    if (r != PXA_OK && rc == PXA_OK) rc = r;
  }
  return rc;
}

int hip_rc(hipError_t e) {
  if (e == hipSuccess) return PXA_OK;
  std::strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = 0;
  return PXA_EHIP;
}

void layout_of(const pxa_config* c, const pxa_options* b, pxa_workspace_layout* L) {
  const pxa::LaunchArgs a = args_of(c, b);
  const size_t nb = (size_t)pxa::num_blocks(a.N);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = pxa::align_up(off + bytes, 256);
    return o;
  };
  L->qbar = take((size_t)a.G * a.N * a.D * 2);
  L->kbar = take((size_t)a.G * a.N * a.D * 2);
  L->scores = take((size_t)a.G * nb * nb * 4);
  L->masses = take((size_t)a.H * nb * 4);
  L->k_h = take((size_t)a.H * 4);
  L->row_ptr = take(((size_t)a.H * nb + 1) * 4);
  L->col_idx = take((size_t)a.H * nb * (nb + 1) / 2 * 4);
  L->row_order = take((size_t)a.H * nb * 4);
  L->budget_ws = take(pxa::budget_ws_bytes(a));
  L->select_ws = take(pxa::select_ws_bytes(a));
  L->total = off;
}

}  // namespace

extern "C" {

int pxa_abi_version(void) { return PXA_ABI_VERSION; }

const char* pxa_strerror(int code) {
  switch (code) {
    case PXA_OK: return "ok";
    case PXA_EINVAL: return "invalid configuration (shape, grouping, gamma, scale or budget)";
    case PXA_EUNSUPPORTED: return "unsupported configuration (head_dim, block, seq_len too large)";
    case PXA_ENULL: return "null pointer";
    case PXA_EALIGN: return "misaligned pointer";
    case PXA_EWORKSPACE: return "workspace too small";
    case PXA_EHIP: return "HIP launch failure";
    default: return "unknown error code";
  }
}

const char* pxa_last_hip_error(void) { return g_last_hip_error; }

int pxa_validate_config(const pxa_config* cfg) { return check_config(cfg); }

size_t pxa_workspace_bytes(const pxa_config* cfg) {
  if (check_config(cfg) != PXA_OK) return 0;
  pxa_workspace_layout L;
  layout_of(cfg, nullptr, &L);
  return L.total;
}

int pxa_get_workspace_layout(const pxa_config* cfg, pxa_workspace_layout* out) {
  const int rc = check_config(cfg);
  if (rc != PXA_OK) return rc;
  if (!out) return PXA_ENULL;
  layout_of(cfg, nullptr, out);
  return PXA_OK;
}

size_t pxa_budget_workspace_bytes(const pxa_config* cfg) {
  if (check_config(cfg) != PXA_OK) return 0;
  return pxa::budget_ws_bytes(args_of(cfg));
}

size_t pxa_select_workspace_bytes(const pxa_config* cfg) {
  if (check_config(cfg) != PXA_OK) return 0;
  return pxa::select_ws_bytes(args_of(cfg));
}

size_t pxa_max_col_entries(const pxa_config* cfg) {
  if (check_config(cfg) != PXA_OK) return 0;
  const size_t nb = (size_t)pxa::num_blocks(cfg->seq_len);
  return (size_t)cfg->num_heads * nb * (nb + 1) / 2;
}

int pxa_validate_options(const pxa_config* cfg, const pxa_options* budget) {
  return check_all(cfg, budget);
}

size_t pxa_workspace_bytes_ex(const pxa_config* cfg, const pxa_options* budget) {
  if (check_all(cfg, budget) != PXA_OK) return 0;
  pxa_workspace_layout L;
  layout_of(cfg, budget, &L);
  return L.total;
}

int pxa_get_workspace_layout_ex(const pxa_config* cfg, const pxa_options* budget,
                                pxa_workspace_layout* out) {
  const int rc = check_all(cfg, budget);
  if (rc != PXA_OK) return rc;
  if (!out) return PXA_ENULL;
  layout_of(cfg, budget, out);
  return PXA_OK;
}

size_t pxa_budget_workspace_bytes_ex(const pxa_config* cfg, const pxa_options* budget) {
  if (check_all(cfg, budget) != PXA_OK) return 0;
  return pxa::budget_ws_bytes(args_of(cfg, budget));
}

int pxa_proxy_pool(const pxa_config* cfg, const void* q, const void* k, void* qbar, void* kbar,
                   void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {qbar, 16}, {kbar, 16}}))) return rc;
  return hip_rc(pxa::launch_proxy_pool(args_of(cfg), q, k, qbar, kbar, (hipStream_t)stream));
}

int pxa_proxy_score_ex(const pxa_config* cfg, const pxa_options* opts, const void* qbar,
                       const void* kbar, float* scores, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = ptrs_ok({{qbar, 16}, {kbar, 16}, {scores, 4}}))) return rc;
  return hip_rc(pxa::launch_proxy_score(args_of(cfg, opts), qbar, kbar, scores,
                                        (hipStream_t)stream));
}

int pxa_proxy_score(const pxa_config* cfg, const void* qbar, const void* kbar, float* scores,
                    void* stream) {
  return pxa_proxy_score_ex(cfg, nullptr, qbar, kbar, scores, stream);
}

int pxa_budget_estimate_ex(const pxa_config* cfg, const pxa_options* budget, const void* q,
                           const void* k, const float* scores, int32_t* k_h, float* masses,
                           void* ws, size_t ws_bytes, void* stream) {
  int rc = check_all(cfg, budget);
  if (rc) return rc;
  const pxa::LaunchArgs a = args_of(cfg, budget);
  if (a.budget_mode == pxa::kBudgetRatio) return PXA_EINVAL;   // no per-head budget
  if (a.budget_mode == pxa::kBudgetFixed) {
    if ((rc = ptrs_ok({{k_h, 4}}))) return rc;
    return hip_rc(pxa::launch_fixed_budget(a, k_h, (hipStream_t)stream));
  }
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {scores, 4}, {k_h, 4}, {masses, 4}, {ws, 256}}))) return rc;
  if (ws_bytes < pxa::budget_ws_bytes(a)) return PXA_EWORKSPACE;
  return hip_rc(pxa::launch_budget(a, q, k, scores, k_h, masses, ws, (hipStream_t)stream));
}

int pxa_budget_estimate(const pxa_config* cfg, const void* q, const void* k, const float* scores,
                        int32_t* k_h, float* masses, void* ws, size_t ws_bytes, void* stream) {
  return pxa_budget_estimate_ex(cfg, nullptr, q, k, scores, k_h, masses, ws, ws_bytes, stream);
}

int pxa_block_select_ex(const pxa_config* cfg, const pxa_options* budget, const float* scores,
                        const int32_t* k_h, int32_t* row_ptr, int32_t* col_idx,
                        int32_t* row_order, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_all(cfg, budget);
  if (rc) return rc;
  const pxa::LaunchArgs a = args_of(cfg, budget);
  const bool ratio = a.budget_mode == pxa::kBudgetRatio;
  if ((rc = ptrs_ok({{scores, 4}, {row_ptr, 4}, {col_idx, 4}, {ws, 256}}))) return rc;
  if (!ratio && (rc = ptrs_ok({{k_h, 4}}))) return rc;
  if (row_order && !aligned(row_order, 4)) return PXA_EALIGN;
  if (ws_bytes < pxa::select_ws_bytes(a)) return PXA_EWORKSPACE;
  return hip_rc(pxa::launch_select(a, scores, ratio ? nullptr : k_h, row_ptr, col_idx, row_order,
                                   ws, (hipStream_t)stream));
}

int pxa_block_select(const pxa_config* cfg, const float* scores, const int32_t* k_h,
                     int32_t* row_ptr, int32_t* col_idx, int32_t* row_order, void* ws,
                     size_t ws_bytes, void* stream) {
  return pxa_block_select_ex(cfg, nullptr, scores, k_h, row_ptr, col_idx, row_order, ws, ws_bytes,
                             stream);
}

int pxa_sparse_prefill_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                          const void* k, const void* v, const int32_t* row_ptr,
                          const int32_t* col_idx, const int32_t* row_order, void* o,
                          void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {row_ptr, 4}, {col_idx, 4}, {o, 16}}))) return rc;
  if (row_order && !aligned(row_order, 4)) return PXA_EALIGN;
  return hip_rc(pxa::launch_fa_prefill(args_of(cfg, opts), q, k, v, row_ptr, col_idx, row_order,
                                       o, false, (hipStream_t)stream));
}

int pxa_sparse_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v,
                       const int32_t* row_ptr, const int32_t* col_idx, const int32_t* row_order,
                       void* o, void* stream) {
  return pxa_sparse_prefill_ex(cfg, nullptr, q, k, v, row_ptr, col_idx, row_order, o, stream);
}

int pxa_dense_prefill_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                         const void* k, const void* v, void* o, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {o, 16}}))) return rc;
  return hip_rc(pxa::launch_fa_prefill(args_of(cfg, opts), q, k, v, nullptr, nullptr, nullptr, o,
                                       true, (hipStream_t)stream));
}

int pxa_dense_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v, void* o,
                      void* stream) {
  return pxa_dense_prefill_ex(cfg, nullptr, q, k, v, o, stream);
}

int pxa_prefill_ex(const pxa_config* cfg, const pxa_options* budget, const void* q,
                   const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check_all(cfg, budget);
  if (rc) return rc;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {o, 16}, {ws, 256}}))) return rc;
  pxa_workspace_layout L;
  layout_of(cfg, budget, &L);
  if (ws_bytes < L.total) return PXA_EWORKSPACE;
  const pxa::LaunchArgs a = args_of(cfg, budget);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  void* qbar = w + L.qbar;
  void* kbar = w + L.kbar;
  float* scores = (float*)(w + L.scores);
  float* masses = (float*)(w + L.masses);
  int32_t* k_h = (int32_t*)(w + L.k_h);
  int32_t* row_ptr = (int32_t*)(w + L.row_ptr);
  int32_t* col_idx = (int32_t*)(w + L.col_idx);
  int32_t* row_order = (int32_t*)(w + L.row_order);
  if ((rc = hip_rc(pxa::launch_proxy_pool(a, q, k, qbar, kbar, s)))) return rc;
  if ((rc = hip_rc(pxa::launch_proxy_score(a, qbar, kbar, scores, s)))) return rc;
  if (a.budget_mode == pxa::kBudgetDynamic)
    rc = hip_rc(pxa::launch_budget(a, q, k, scores, k_h, masses, w + L.budget_ws, s));
  else if (a.budget_mode == pxa::kBudgetFixed)
    rc = hip_rc(pxa::launch_fixed_budget(a, k_h, s));
  if (rc) return rc;
  const bool ratio = a.budget_mode == pxa::kBudgetRatio;
  if ((rc = hip_rc(pxa::launch_select(a, scores, ratio ? nullptr : k_h, row_ptr, col_idx,
                                      row_order, w + L.select_ws, s))))
    return rc;
  return hip_rc(pxa::launch_fa_prefill(a, q, k, v, row_ptr, col_idx, row_order, o, false, s));
}

int pxa_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v, void* o,
                void* ws, size_t ws_bytes, void* stream) {
  return pxa_prefill_ex(cfg, nullptr, q, k, v, o, ws, ws_bytes, stream);
}

int pxa_prefill_batch(const pxa_config* cfg, const pxa_options* opts, int32_t num_seqs,
                      const int32_t* seq_lens, const void* q, const void* k, const void* v,
                      void* o, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if (num_seqs < 1) return PXA_EINVAL;
  if (!seq_lens) return PXA_ENULL;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {o, 16}, {ws, 256}}))) return rc;
  if (ws_bytes < pxa_workspace_bytes_ex(cfg, opts)) return PXA_EWORKSPACE;
  for (int32_t s = 0; s < num_seqs; ++s) {   // validate every length before any launch
    const int32_t n = seq_lens[s];
    if (n < 1 || n > cfg->seq_len) return PXA_EINVAL;
    pxa_config c = *cfg;
    c.seq_len = n;
    if ((rc = check_all(&c, opts))) return rc;   // e.g. a probe longer than this sequence
  }
  const size_t qrow = (size_t)cfg->num_heads * cfg->head_dim * 2;      // bytes per token
  const size_t krow = (size_t)cfg->num_kv_heads * cfg->head_dim * 2;
  size_t qoff = 0, koff = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    pxa_config c = *cfg;
    c.seq_len = seq_lens[s];
    rc = pxa_prefill_ex(&c, opts, (const char*)q + qoff, (const char*)k + koff,
                        (const char*)v + koff, (char*)o + qoff, ws, ws_bytes, stream);
    if (rc) return rc;
    qoff += qrow * (size_t)c.seq_len;
    koff += krow * (size_t)c.seq_len;
  }
  return PXA_OK;
}

}  // extern "C"
