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

// The sequences one set of launches covers (one, or a fused batch of up to
// kMaxFusedSeqs), stored one after another: the tensors of sequence s
// (Q/O [H][N_s][d], K/V [Hkv][N_s][d]) follow those of sequences 0..s-1, and
// so do its intermediates in every workspace part (proxies, scores, masses,
// k_h, the CSR rows and the stage scratch).  Prefix sums over the sequences
// before s; passed by value, so the kernels read them from the kernel
// argument segment (scalar loads, no copy).
constexpr int kMaxFusedSeqs = 64;
struct SeqTable {
  int32_t n;                        // sequences
  int32_t tok[kMaxFusedSeqs + 1];   // tokens
  int32_t blk[kMaxFusedSeqs + 1];   // blocks, nb_t = ceil(N_t / 128)
  int32_t sq[kMaxFusedSeqs + 1];    // nb_t^2: score entries per proxy
  int32_t swg[kMaxFusedSeqs + 1];   // score workgroups, G * ceil(nb_t / stride)
};

// lens[0..n-1] (1 <= n <= kMaxFusedSeqs), each >= 1; sums are checked by the caller.
inline SeqTable make_table(const int32_t* lens, int n, int G, int stride) {
  SeqTable t{};
  t.n = n;
  for (int s = 0; s < n; ++s) {
    const int nb = num_blocks(lens[s]);
    t.tok[s + 1] = t.tok[s] + lens[s];
    t.blk[s + 1] = t.blk[s] + nb;
    t.sq[s + 1] = t.sq[s] + nb * nb;
    t.swg[s + 1] = t.swg[s] + G * ((nb + stride - 1) / stride);
  }
  return t;
}
inline SeqTable one_seq(const LaunchArgs& a) {
  const int32_t n = a.N;
  return make_table(&n, 1, a.G, a.score_stride);
}
inline int max_len(const SeqTable& t) {
  int m = 0;
  for (int s = 0; s < t.n; ++s) m = t.tok[s + 1] - t.tok[s] > m ? t.tok[s + 1] - t.tok[s] : m;
  return m;
}
inline int max_blocks(const SeqTable& t) { return num_blocks(max_len(t)); }

// proxies: fp16 [G][N][d] per sequence, block exponents int32 [G][nb] per sequence
hipError_t launch_proxy_pool(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                             void* qbar, void* kbar, int32_t* qexp, int32_t* kexp,
                             hipStream_t stream);
hipError_t launch_proxy_score(const LaunchArgs& a, const SeqTable& t, const void* qbar,
                              const void* kbar, const int32_t* qexp, const int32_t* kexp,
                              float* scores, hipStream_t stream);
// ws: budget_ws_bytes(a, t) bytes
size_t budget_ws_bytes(const LaunchArgs& a, const SeqTable& t);
hipError_t launch_budget(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                         const float* scores, int32_t* k_h, float* masses, void* ws,
                         hipStream_t stream);
// fixed budget: k_h[s][h] = a.fixed_blocks
hipError_t launch_fixed_budget(const LaunchArgs& a, const SeqTable& t, int32_t* k_h,
                               hipStream_t stream);
// ws: select_ws_bytes(a, t) bytes
size_t select_ws_bytes(const LaunchArgs& a, const SeqTable& t);
// k_h NULL: the ratio budget a.ratio
hipError_t launch_select(const LaunchArgs& a, const SeqTable& t, const float* scores,
                         const int32_t* k_h, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* row_order, void* ws, hipStream_t stream);
hipError_t launch_fa_prefill(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                             const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* row_order, void* o, bool dense, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace pxa
