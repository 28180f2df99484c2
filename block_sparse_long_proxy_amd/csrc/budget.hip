// budget.hip -- block-aware dynamic budget per head.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 2: the last small part
// of the query blocks estimates each head's block-level sparsity, so heads
// that share one importance ranking get different block budgets.  Reading:
// the probe is every query of the last m query blocks (m = 1 by default: 128
// queries, fewer when the last block is partial);
// each probe query's exact causal softmax; masses[h][J] = mean over the probe
// queries of the probability mass in key block J; k_h = fewest leading blocks
// of the group's ranking of row nb-1 (score descending, block ascending on
// ties) whose masses reach gamma, else nb.  The fixed budget that step is
// compared with sets k_h to one value for every head (budget_fixed_kernel).
//
// Kernel 1 (budget_lse_kernel): one workgroup per (head, run of key blocks,
//   probe block); key tiles stream through a two-deep LDS ring filled by
//   direct copies; for each causal key block J the 128x128 logit tile
//   S^T = K_J Q_T^T (MFMA) is reduced to a per-query log2-sum-exp2 over that
//   block, lse[h][z][J][i].
// Kernel 2 (budget_finalize_kernel): one workgroup per (sequence, head); per probe block,
//   merges the partials into each query's normaliser and adds the block
//   masses; then sorts the last row's scores in LDS (bitonic, 64-bit keys)
//   and scans the masses in rank order (fp32, fixed chunked order) for k_h.
#include <type_traits>

#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kLseBlocksPerWG = 8;
constexpr int kFinThreads = 512;

template <int D>
__global__ __launch_bounds__(kThreads, 2) void budget_lse_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, float* __restrict__ lse,
    int H, int Hkv, int m, float scale_log2, const SeqTable t) {
  // two-deep ring of K tiles, filled by direct global -> LDS copies (tile J+1
  // lands while J is used)
  __shared__ __attribute__((aligned(16))) __bf16 ks[2][kBlock * D];
  const int sid = (int)blockIdx.z / m;     // sequence of a fused batch
  const int z = (int)blockIdx.z % m;       // probe block z of m
  const int N = t.tok[sid + 1] - t.tok[sid];
  const int nb = t.blk[sid + 1] - t.blk[sid];
  q += (size_t)t.tok[sid] * H * D;
  k += (size_t)t.tok[sid] * Hkv * D;
  lse += (size_t)H * m * t.blk[sid] * kBlock;
  const int h = blockIdx.y;
  const int kvh = h / (H / Hkv);
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int qloc = 32 * w + (l & 31);
  const int I = nb - m + z;                // its query block

  const int j0 = blockIdx.x * kLseBlocksPerWG;   // grid x covers the longest sequence
  const int j1 = min(I + 1, j0 + kLseBlocksPerWG);   // causal key blocks only
  if (j0 >= j1) return;
  bf16x8 qf[D / 16];
  // rows past a partial last block repeat token N-1 (excluded from the masses)
  load_qfrag<D>(q + ((size_t)h * N + (size_t)min(I * kBlock + qloc, N - 1)) * D, qf);
  const __bf16* kb = uniform_ptr(k + (size_t)kvh * N * D);
  float* out = lse + ((size_t)h * m + z) * nb * kBlock;
  auto load = [&](int J, __bf16* buf) {   // only block nb-1 can be partial
    const int rows = min(kBlock, N - J * kBlock);
    if (rows < kBlock) tile_load_lds_rows<D, false>(kb + (size_t)J * kBlock * D, buf, rows);
    else tile_load_lds<D, false>(kb + (size_t)J * kBlock * D, buf);
  };
  load(j0, ks[0]);

  // One key block; DIAG: J is the probe block itself (causal mask), which can
  // only be the last block of this workgroup, so the mask stays out of the loop.
  auto step = [&](int J, auto diag_c) {
    constexpr bool DIAG = decltype(diag_c)::value;
    wait_vmem();       // this thread's part of tile J (and the query fragments)
    __syncthreads();   // tile J visible; tile J-1's buffer is no longer read
    if (J + 1 < j1) load(J + 1, ks[(J + 1 - j0) & 1]);
    f32x16 s[4];
    tile_scores<D>(ks[(J - j0) & 1], qf, s);
    if (DIAG) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key(t, r) > qloc) s[t][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // The diagonal block always holds key j = i, so mx is finite.
    const float mb = mx * scale_log2;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)   // v_exp_f32 directly: terms below 2^-126 flush to 0
        sum += __builtin_amdgcn_exp2f(fmaf(s[t][r], scale_log2, -mb));
    sum += __shfl_xor(sum, 32, 64);
    if (l < 32) out[(size_t)J * kBlock + qloc] = mb + log2f(sum);
  };
  for (int J = j0; J < j1 - 1; ++J) step(J, std::false_type{});
  if (j1 - 1 == I) step(I, std::true_type{});
  else step(j1 - 1, std::false_type{});
}

__device__ __forceinline__ void bitonic_sort_u64(uint64_t* keys, int P) {
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int b = a + j;
        const uint64_t x = keys[a], y = keys[b];
        const bool up = (a & kk) == 0;
        if ((x > y) == up) {
          keys[a] = y;
          keys[b] = x;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kFinThreads) void budget_finalize_kernel(
    const float* __restrict__ lse, const float* __restrict__ scores, int32_t* __restrict__ k_h,
    float* __restrict__ masses, int H, int G, int m, float gamma, const SeqTable st) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int sid = (int)blockIdx.x / H;     // sequence of a fused batch
  const int nb = st.blk[sid + 1] - st.blk[sid];
  const int tail = (st.tok[sid + 1] - st.tok[sid]) - (nb - 1) * kBlock;
  lse += (size_t)H * m * st.blk[sid] * kBlock;
  scores += (size_t)G * st.sq[sid];
  masses += (size_t)H * st.blk[sid];
  k_h += (size_t)H * sid;
  int P = 1;                               // sort size: a power of two >= nb
  while (P < nb) P <<= 1;
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);              // [P]
  float* mass = reinterpret_cast<float*>(keys + P);                 // [nb]
  float* qlse = mass + nb;                                          // [128]
  float* part_l = qlse + kBlock;                                    // [4][128]
  float* part_s = part_l + 4 * kBlock;                              // [4][128]
  float* csum = part_s + 4 * kBlock;                                // [kFinThreads]
  __shared__ int first_hit;

  const int h = (int)blockIdx.x % H;
  const int g = h / (H / G);
  const int t = threadIdx.x;

  // 3a. sort keys of the group's last row (loaded first, sorted below).
  const float* srow = scores + ((size_t)g * nb + (nb - 1)) * nb;
  for (int J = t; J < P; J += kFinThreads)
    keys[J] = J < nb ? rank_key(srow[J], (uint32_t)J) : ~0ull;
  for (int J = t; J < nb; J += kFinThreads) mass[J] = 0.f;
  if (t == 0) first_hit = nb;

  for (int z = 0; z < m; ++z) {            // probe blocks, in order
    const int I = nb - m + z;              // causal key blocks 0..I
    const float* L = lse + ((size_t)h * m + z) * nb * kBlock;
    // 1. per-query normaliser (log2 domain), 4 partial merges per query; the
    //    partials of 8 blocks are loaded together (the loop is load-latency
    //    bound otherwise), then folded in with one rescale.
    {
      const int i = t % kBlock, part = t / kBlock;   // kFinThreads == 4 * 128
      float mx = -INFINITY, sm = 0.f;
      auto fold = [&](float x) {
        if (x > mx) {
          sm = sm * exp2f(mx - x) + 1.f;
          mx = x;
        } else {
          sm += exp2f(x - mx);
        }
      };
      int J = part;
      for (; J + 28 <= I; J += 32) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = L[(size_t)(J + 4 * u) * kBlock + i];
        float mloc = x[0];
#pragma unroll
        for (int u = 1; u < 8; ++u) mloc = fmaxf(mloc, x[u]);
        if (mloc > mx) {
          sm = (mx == -INFINITY) ? 0.f : sm * exp2f(mx - mloc);
          mx = mloc;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) sm += exp2f(x[u] - mx);
      }
      for (; J <= I; J += 4) fold(L[(size_t)J * kBlock + i]);
      part_l[part * kBlock + i] = mx;
      part_s[part * kBlock + i] = sm;
    }
    __syncthreads();
    if (t < kBlock) {
      float mx = -INFINITY;
      for (int p = 0; p < 4; ++p) mx = fmaxf(mx, part_l[p * kBlock + t]);
      float sm = 0.f;
      for (int p = 0; p < 4; ++p) {
        const float lp = part_l[p * kBlock + t];
        if (lp != -INFINITY) sm += part_s[p * kBlock + t] * exp2f(lp - mx);
      }
      qlse[t] = mx + log2f(sm);
    }
    __syncthreads();
    // 2. block masses: one wave per block J, lanes over the 128 queries (only
    //    the `rows` that exist in a partial last block).
    {
      const int wv = t >> 6, ln = t & 63, nw = kFinThreads / 64;
      const int rows = I == nb - 1 ? tail : kBlock;
      // a query past a partial last block contributes nothing (its lse is
      // replaced by +inf, so its exponentials are 0)
      const float q0 = ln < rows ? qlse[ln] : INFINITY;
      const float q1 = ln + 64 < rows ? qlse[ln + 64] : INFINITY;
      int J = wv;
      for (; J + 3 * nw <= I; J += 4 * nw) {   // four blocks' loads in flight together
        float a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float* r = L + (size_t)(J + u * nw) * kBlock;
          a[u] = r[ln];
          b[u] = r[ln + 64];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float v = wave_sum(exp2f(a[u] - q0) + exp2f(b[u] - q1));
          if (ln == 0) mass[J + u * nw] += v;
        }
      }
      for (; J <= I; J += nw) {
        const float* r = L + (size_t)J * kBlock;
        const float v = wave_sum(exp2f(r[ln] - q0) + exp2f(r[ln + 64] - q1));
        if (ln == 0) mass[J] += v;
      }
    }
    __syncthreads();   // qlse / part arrays are reused by the next probe block
  }
  {
    const float inv = 1.0f / (float)((m - 1) * kBlock + tail);   // probe queries
    for (int J = t; J < nb; J += kFinThreads) {
      mass[J] *= inv;
      masses[(size_t)h * nb + J] = mass[J];
    }
  }
  // 3b. ranking of row nb-1.
  bitonic_sort_u64(keys, P);   // ends with a barrier

  // 4. cumulative mass in rank order: contiguous chunk per thread.
  const int per = (nb + kFinThreads - 1) / kFinThreads;
  const int r0 = min(nb, t * per), r1 = min(nb, r0 + per);
  float own = 0.f;
  for (int r = r0; r < r1; ++r) own += mass[(uint32_t)keys[r]];
  csum[t] = own;
  __syncthreads();
  if (t == 0) {   // exclusive scan of the chunk sums (sequential, fixed order)
    float run = 0.f;
    for (int i = 0; i < kFinThreads; ++i) {
      const float x = csum[i];
      csum[i] = run;
      run += x;
    }
  }
  __syncthreads();
  float cum = csum[t];
  for (int r = r0; r < r1; ++r) {
    cum += mass[(uint32_t)keys[r]];
    if (cum >= gamma) {
      atomicMin(&first_hit, r);
      break;
    }
  }
  __syncthreads();
  if (t == 0) k_h[h] = first_hit < nb ? first_hit + 1 : nb;
}

static int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

size_t budget_ws_bytes(const LaunchArgs& a, const SeqTable& t) {   // lse [s][H][m][nb_s][128]
  const size_t m = a.budget_mode == kBudgetDynamic ? (size_t)a.last_blocks : 1;
  return align_up((size_t)a.H * m * t.blk[t.n] * kBlock * sizeof(float), 256);
}

__global__ void budget_fixed_kernel(int32_t* __restrict__ k_h, int n, int k) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    k_h[i] = k;
}

hipError_t launch_fixed_budget(const LaunchArgs& a, const SeqTable& t, int32_t* k_h,
                               hipStream_t stream) {
  const int n = a.H * t.n;
  hipLaunchKernelGGL(budget_fixed_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, k_h, n,
                     a.fixed_blocks);
  return hipGetLastError();
}

hipError_t launch_budget(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                         const float* scores, int32_t* k_h, float* masses, void* ws,
                         hipStream_t stream) {
  const int nb = max_blocks(t);
  float* lse = (float*)ws;
  const float sl2 = a.scale * kLog2e;
  const int m = a.last_blocks;
  const dim3 g1((nb + kLseBlocksPerWG - 1) / kLseBlocksPerWG, a.H, m * t.n);
  if (a.D == 64)
    hipLaunchKernelGGL(budget_lse_kernel<64>, g1, dim3(kThreads), 0, stream, (const __bf16*)q,
                       (const __bf16*)k, lse, a.H, a.Hkv, m, sl2, t);
  else
    hipLaunchKernelGGL(budget_lse_kernel<128>, g1, dim3(kThreads), 0, stream, (const __bf16*)q,
                       (const __bf16*)k, lse, a.H, a.Hkv, m, sl2, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = pow2_at_least(nb);   // LDS for the longest sequence
  const size_t smem = (size_t)P * 8 + (size_t)nb * 4 + (size_t)kBlock * 4 * 9 + kFinThreads * 4;
  hipLaunchKernelGGL(budget_finalize_kernel, dim3(a.H * t.n), dim3(kFinThreads), smem, stream, lse,
                     scores, k_h, masses, a.H, a.G, m, a.gamma, t);
  return hipGetLastError();
}

}  // namespace pxa
