// pxa_abi.cpp -- the extern "C" boundary (include/pxa.h): host-side
// validation, workspace layout and the launch sequence.  No allocation, no
// synchronisation, no global mutable state except a thread-local copy of the
// last HIP error message and, for pxa_prefill_noalloc only, the per-device
// address of the library's static scratch array.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
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

// Workspace parts of one set of launches over the sequences of t, each part
// the concatenation of the sequences' own parts in order.
void layout_of_table(const pxa::LaunchArgs& a, const pxa::SeqTable& t, pxa_workspace_layout* L) {
  const size_t toks = (size_t)t.tok[t.n], blks = (size_t)t.blk[t.n], sq = (size_t)t.sq[t.n];
  size_t tri = 0;   // causal blocks of one head, summed over the sequences
  for (int s = 0; s < t.n; ++s) {
    const size_t nb = (size_t)(t.blk[s + 1] - t.blk[s]);
    tri += nb * (nb + 1) / 2;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = pxa::align_up(off + bytes, 256);
    return o;
  };
  L->qbar = take((size_t)a.G * toks * a.D * 2);
  L->kbar = take((size_t)a.G * toks * a.D * 2);
  L->qexp = take((size_t)a.G * blks * 4);
  L->kexp = take((size_t)a.G * blks * 4);
  L->scores = take((size_t)a.G * sq * 4);
  L->masses = take((size_t)a.H * blks * 4);
  L->k_h = take((size_t)a.H * t.n * 4);
  L->row_ptr = take(((size_t)a.H * blks + 1) * 4);
  L->col_idx = take((size_t)a.H * tri * 4);
  L->row_order = take((size_t)a.H * blks * 4);
  L->budget_ws = take(pxa::budget_ws_bytes(a, t));
  L->select_ws = take(pxa::select_ws_bytes(a, t));
  L->total = off;
}

void layout_of(const pxa_config* c, const pxa_options* b, pxa_workspace_layout* L) {
  const pxa::LaunchArgs a = args_of(c, b);
  layout_of_table(a, pxa::one_seq(a), L);
}

// The whole method over the sequences of t on one stream (workspace laid out
// by layout_of_table).
int run_method(const pxa::LaunchArgs& a, const pxa::SeqTable& t, const void* q, const void* k,
               const void* v, void* o, void* ws, const pxa_workspace_layout& L,
               hipStream_t s) {
  char* w = (char*)ws;
  void* qbar = w + L.qbar;
  void* kbar = w + L.kbar;
  int32_t* qexp = (int32_t*)(w + L.qexp);
  int32_t* kexp = (int32_t*)(w + L.kexp);
  float* scores = (float*)(w + L.scores);
  float* masses = (float*)(w + L.masses);
  int32_t* k_h = (int32_t*)(w + L.k_h);
  int32_t* row_ptr = (int32_t*)(w + L.row_ptr);
  int32_t* col_idx = (int32_t*)(w + L.col_idx);
  int32_t* row_order = (int32_t*)(w + L.row_order);
  int rc;
  if ((rc = hip_rc(pxa::launch_proxy_pool(a, t, q, k, qbar, kbar, qexp, kexp, s)))) return rc;
  if ((rc = hip_rc(pxa::launch_proxy_score(a, t, qbar, kbar, qexp, kexp, scores, s)))) return rc;
  if (a.budget_mode == pxa::kBudgetDynamic)
    rc = hip_rc(pxa::launch_budget(a, t, q, k, scores, k_h, masses, w + L.budget_ws, s));
  else if (a.budget_mode == pxa::kBudgetFixed)
    rc = hip_rc(pxa::launch_fixed_budget(a, t, k_h, s));
  if (rc) return rc;
  const bool ratio = a.budget_mode == pxa::kBudgetRatio;
  if ((rc = hip_rc(pxa::launch_select(a, t, scores, ratio ? nullptr : k_h, row_ptr, col_idx,
                                      row_order, w + L.select_ws, s))))
    return rc;
  return hip_rc(pxa::launch_fa_prefill(a, t, q, k, v, row_ptr, col_idx, row_order, o, false, s));
}

// Groups of a batch fused into one set of launches: consecutive sequences,
// at most kMaxFusedSeqs of them, with all CSR entries of a group addressable
// by int32.  Calls f(first, count) for each group in order.
template <typename F>
void for_each_group(const pxa_config* c, int32_t n, const int32_t* lens, F&& f) {
  int32_t first = 0;
  while (first < n) {
    int32_t cnt = 0;
    int64_t entries = 0;
    while (first + cnt < n && cnt < pxa::kMaxFusedSeqs) {
      const int64_t nb = pxa::num_blocks(lens[first + cnt]);
      const int64_t add = (int64_t)c->num_heads * nb * (nb + 1) / 2;
      if (cnt > 0 && entries + add > INT32_MAX) break;
      entries += add;
      ++cnt;
    }
    f(first, cnt);
    first += cnt;
  }
}

// Lengths of a batch: every one valid for cfg and opts (PXA_OK) or the first error.
int check_lengths(const pxa_config* cfg, const pxa_options* opts, int32_t n, const int32_t* lens) {
  if (n < 1) return PXA_EINVAL;
  if (!lens) return PXA_ENULL;
  for (int32_t s = 0; s < n; ++s) {
    if (lens[s] < 1 || lens[s] > cfg->seq_len) return PXA_EINVAL;
    pxa_config c = *cfg;
    c.seq_len = lens[s];
    const int rc = check_all(&c, opts);   // e.g. a probe longer than this sequence
    if (rc) return rc;
  }
  return PXA_OK;
}

size_t fused_bytes(const pxa_config* cfg, const pxa_options* opts, int32_t n, const int32_t* lens) {
  const pxa::LaunchArgs a = args_of(cfg, opts);
  size_t need = 0;
  for_each_group(cfg, n, lens, [&](int32_t first, int32_t cnt) {
    pxa_workspace_layout L;
    layout_of_table(a, pxa::make_table(lens + first, cnt, a.G, a.score_stride), &L);
    need = L.total > need ? L.total : need;
  });
  return need;
}

// Workspace of pxa_prefill_noalloc: one array per GPU, held from the moment
// the library's code object is loaded on that GPU until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in symbol): the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) unsigned char scratch[PXA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call for that device), or the PXA_E* code of a failure.
int scratch_of_current_device(void** out) {
  int dev = -1;
  int rc = hip_rc(hipGetDevice(&dev));
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices) return PXA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((rc = hip_rc(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))))) return rc;
    if (!ptr || !aligned(ptr, 256)) return PXA_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PXA_OK;
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
  const pxa::LaunchArgs a = args_of(cfg);
  return pxa::budget_ws_bytes(a, pxa::one_seq(a));
}

size_t pxa_select_workspace_bytes(const pxa_config* cfg) {
  if (check_config(cfg) != PXA_OK) return 0;
  const pxa::LaunchArgs a = args_of(cfg);
  return pxa::select_ws_bytes(a, pxa::one_seq(a));
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
  const pxa::LaunchArgs a = args_of(cfg, budget);
  return pxa::budget_ws_bytes(a, pxa::one_seq(a));
}

int pxa_proxy_pool(const pxa_config* cfg, const void* q, const void* k, void* qbar, void* kbar,
                   int32_t* qexp, int32_t* kexp, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {qbar, 16}, {kbar, 16}, {qexp, 4}, {kexp, 4}}))) return rc;
  const pxa::LaunchArgs a = args_of(cfg);
  return hip_rc(pxa::launch_proxy_pool(a, pxa::one_seq(a), q, k, qbar, kbar, qexp, kexp,
                                       (hipStream_t)stream));
}

int pxa_proxy_score_ex(const pxa_config* cfg, const pxa_options* opts, const void* qbar,
                       const void* kbar, const int32_t* qexp, const int32_t* kexp,
                       float* scores, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = ptrs_ok({{qbar, 16}, {kbar, 16}, {qexp, 4}, {kexp, 4}, {scores, 4}}))) return rc;
  const pxa::LaunchArgs a = args_of(cfg, opts);
  return hip_rc(pxa::launch_proxy_score(a, pxa::one_seq(a), qbar, kbar, qexp, kexp, scores,
                                        (hipStream_t)stream));
}

int pxa_proxy_score(const pxa_config* cfg, const void* qbar, const void* kbar,
                    const int32_t* qexp, const int32_t* kexp, float* scores, void* stream) {
  return pxa_proxy_score_ex(cfg, nullptr, qbar, kbar, qexp, kexp, scores, stream);
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
    return hip_rc(pxa::launch_fixed_budget(a, pxa::one_seq(a), k_h, (hipStream_t)stream));
  }
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {scores, 4}, {k_h, 4}, {masses, 4}, {ws, 256}}))) return rc;
  const pxa::SeqTable t = pxa::one_seq(a);
  if (ws_bytes < pxa::budget_ws_bytes(a, t)) return PXA_EWORKSPACE;
  return hip_rc(pxa::launch_budget(a, t, q, k, scores, k_h, masses, ws, (hipStream_t)stream));
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
  const pxa::SeqTable t = pxa::one_seq(a);
  if (ws_bytes < pxa::select_ws_bytes(a, t)) return PXA_EWORKSPACE;
  return hip_rc(pxa::launch_select(a, t, scores, ratio ? nullptr : k_h, row_ptr, col_idx,
                                   row_order, ws, (hipStream_t)stream));
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
  const pxa::LaunchArgs a = args_of(cfg, opts);
  return hip_rc(pxa::launch_fa_prefill(a, pxa::one_seq(a), q, k, v, row_ptr, col_idx, row_order,
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
  const pxa::LaunchArgs a = args_of(cfg, opts);
  return hip_rc(pxa::launch_fa_prefill(a, pxa::one_seq(a), q, k, v, nullptr, nullptr, nullptr, o,
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
  return run_method(a, pxa::one_seq(a), q, k, v, o, ws, L, (hipStream_t)stream);
}

int pxa_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v, void* o,
                void* ws, size_t ws_bytes, void* stream) {
  return pxa_prefill_ex(cfg, nullptr, q, k, v, o, ws, ws_bytes, stream);
}

int pxa_prefill_noalloc(const pxa_config* cfg, const pxa_options* opts, const void* q,
                        const void* k, const void* v, void* o, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  pxa_workspace_layout L;
  layout_of(cfg, opts, &L);
  if (L.total > PXA_NOALLOC_SCRATCH_BYTES) return PXA_EWORKSPACE;   // before any HIP call
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {o, 16}}))) return rc;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  const pxa::LaunchArgs a = args_of(cfg, opts);
  return run_method(a, pxa::one_seq(a), q, k, v, o, ws, L, (hipStream_t)stream);
}

size_t pxa_batch_workspace_bytes(const pxa_config* cfg, const pxa_options* opts,
                                 int32_t num_seqs, const int32_t* seq_lens) {
  if (check_all(cfg, opts) != PXA_OK) return 0;
  if (check_lengths(cfg, opts, num_seqs, seq_lens) != PXA_OK) return 0;
  return fused_bytes(cfg, opts, num_seqs, seq_lens);
}

int pxa_get_batch_workspace_layout(const pxa_config* cfg, const pxa_options* opts,
                                   int32_t num_seqs, const int32_t* seq_lens,
                                   pxa_workspace_layout* out) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = check_lengths(cfg, opts, num_seqs, seq_lens))) return rc;
  if (!out) return PXA_ENULL;
  int groups = 0;
  for_each_group(cfg, num_seqs, seq_lens, [&](int32_t, int32_t) { ++groups; });
  if (groups != 1) return PXA_EINVAL;   // more than one fused group
  const pxa::LaunchArgs a = args_of(cfg, opts);
  layout_of_table(a, pxa::make_table(seq_lens, num_seqs, a.G, a.score_stride), out);
  return PXA_OK;
}

int pxa_prefill_batch(const pxa_config* cfg, const pxa_options* opts, int32_t num_seqs,
                      const int32_t* seq_lens, const void* q, const void* k, const void* v,
                      void* o, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_all(cfg, opts);
  if (rc) return rc;
  if ((rc = check_lengths(cfg, opts, num_seqs, seq_lens))) return rc;   // before any launch
  if ((rc = ptrs_ok({{q, 16}, {k, 16}, {v, 16}, {o, 16}, {ws, 256}}))) return rc;
  const pxa::LaunchArgs a = args_of(cfg, opts);
  const size_t qrow = (size_t)cfg->num_heads * cfg->head_dim * 2;      // bytes per token
  const size_t krow = (size_t)cfg->num_kv_heads * cfg->head_dim * 2;
  hipStream_t st = (hipStream_t)stream;
  if (ws_bytes >= fused_bytes(cfg, opts, num_seqs, seq_lens)) {
    // fused: one set of launches per group of sequences
    size_t tok = 0;
    for_each_group(cfg, num_seqs, seq_lens, [&](int32_t first, int32_t cnt) {
      if (rc) return;
      const pxa::SeqTable t = pxa::make_table(seq_lens + first, cnt, a.G, a.score_stride);
      pxa_workspace_layout L;
      layout_of_table(a, t, &L);
      rc = run_method(a, t, (const char*)q + qrow * tok, (const char*)k + krow * tok,
                      (const char*)v + krow * tok, (char*)o + qrow * tok, ws, L, st);
      tok += (size_t)t.tok[t.n];
    });
    return rc;
  }
  // sequence by sequence in a workspace sized for the longest one
  if (ws_bytes < pxa_workspace_bytes_ex(cfg, opts)) return PXA_EWORKSPACE;
  size_t tok = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    pxa_config c = *cfg;
    c.seq_len = seq_lens[s];
    rc = pxa_prefill_ex(&c, opts, (const char*)q + qrow * tok, (const char*)k + krow * tok,
                        (const char*)v + krow * tok, (char*)o + qrow * tok, ws, ws_bytes, stream);
    if (rc) return rc;
    tok += (size_t)c.seq_len;
  }
  return PXA_OK;
}

}  // extern "C"
