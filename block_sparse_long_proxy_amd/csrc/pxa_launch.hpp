// pxa_launch.hpp -- host-side launch interface between the C ABI layer and
// the kernel files.  Arguments are validated by the ABI layer before any of
// these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pxa {

constexpr int kBlockTokens = 128;   // block edge the kernels are built for

// Blocks of a sequence of N tokens; the last one is partial when 128 does not
// divide N (its missing rows are read as copies of token N-1 and never written).
inline int num_blocks(int N) { return (N + kBlockTokens - 1) / kBlockTokens; }

enum BudgetMode { kBudgetDynamic = 0, kBudgetFixed = 1, kBudgetRatio = 2 };

struct LaunchArgs {
  int H, Hkv, N, D, G;
  float scale;   // softmax scale (already defaulted)
  float gamma;
  int budget_mode = kBudgetDynamic;
  int last_blocks = 1;    // dynamic budget: query blocks probed
  int fixed_blocks = 0;   // fixed budget: blocks per row
  float ratio = 0.f;      // ratio budget
  int score_stride = 1;   // queries scored per block: 128 / score_stride
  float skip_threshold = 0.f;   // running-max skip of the attention (0: off)
};

hipError_t launch_proxy_pool(const LaunchArgs& a, const void* q, const void* k, void* qbar,
                             void* kbar, hipStream_t stream);
hipError_t launch_proxy_score(const LaunchArgs& a, const void* qbar, const void* kbar,
                              float* scores, hipStream_t stream);
// ws: budget_ws_bytes(a) bytes
size_t budget_ws_bytes(const LaunchArgs& a);
hipError_t launch_budget(const LaunchArgs& a, const void* q, const void* k, const float* scores,
                         int32_t* k_h, float* masses, void* ws, hipStream_t stream);
// fixed budget: k_h[h] = a.fixed_blocks
hipError_t launch_fixed_budget(const LaunchArgs& a, int32_t* k_h, hipStream_t stream);
// ws: select_ws_bytes(a) bytes
size_t select_ws_bytes(const LaunchArgs& a);
// k_h NULL: the ratio budget a.ratio
hipError_t launch_select(const LaunchArgs& a, const float* scores, const int32_t* k_h,
                         int32_t* row_ptr, int32_t* col_idx, int32_t* row_order, void* ws,
                         hipStream_t stream);
hipError_t launch_fa_prefill(const LaunchArgs& a, const void* q, const void* k, const void* v,
                             const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* row_order, void* o, bool dense, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace pxa
