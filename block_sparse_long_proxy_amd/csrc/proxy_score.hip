// proxy_score.hip -- fused proxy QK^T + 128x128 block max-pool.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Score Estimation":
// token-level scores of the proxy head are max-pooled into block importance
// scores, with the QK product and the max pooling fused at block level.
// Causal prefill: in the diagonal block only keys j <= i count; blocks above
// the diagonal get -inf.
//
// One workgroup per (proxy g, query block I), 4 waves x 32 queries, proxy
// queries held as MFMA B operands in registers; key tiles J = 0..I stream
// through LDS.  The max is taken in registers, across the wave with shuffles
// and across the 4 waves through a double-buffered LDS slot, so each tile
// costs one barrier.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

template <int D>
__global__ __launch_bounds__(kThreads, 2) void proxy_score_kernel(
    const __bf16* __restrict__ qbar, const __bf16* __restrict__ kbar, float* __restrict__ scores,
    int G, int N, float scale) {
  __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * D];
  __shared__ float wmax[2][kWaves];

  const int nb = N / kBlock;
  const int I = nb - 1 - (int)(blockIdx.x / G);
  const int g = (int)(blockIdx.x % G);
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int qloc = 32 * w + (l & 31);

  bf16x8 qf[D / 16];
  load_qfrag<D>(qbar + ((size_t)g * N + (size_t)I * kBlock + qloc) * D, qf);
  const __bf16* kb = kbar + (size_t)g * N * D;
  float* srow = scores + ((size_t)g * nb + I) * nb;

  for (int J = I + 1 + threadIdx.x; J < nb; J += kThreads) srow[J] = -INFINITY;

  for (int J = 0; J <= I; ++J) {
    __syncthreads();
    if (J > 0 && threadIdx.x == 0) {
      const float* wm = wmax[(J - 1) & 1];
      srow[J - 1] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])) * scale;
    }
    stage_ktile<D>(kb + (size_t)J * kBlock * D, ks);
    __syncthreads();

    f32x16 s[4];
    tile_scores<D>(ks, qf, s);
    float mx = -INFINITY;
    if (J == I) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key(t, r) <= qloc) mx = fmaxf(mx, s[t][r]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    }
    mx = wave_max(mx);
    if (l == 0) wmax[J & 1][w] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float* wm = wmax[I & 1];
    srow[I] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])) * scale;
  }
}

hipError_t launch_proxy_score(const LaunchArgs& a, const void* qbar, const void* kbar,
                              float* scores, hipStream_t stream) {
  const dim3 grid(a.G * (a.N / kBlock)), block(kThreads);
  if (a.D == 64)
    hipLaunchKernelGGL(proxy_score_kernel<64>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  else
    hipLaunchKernelGGL(proxy_score_kernel<128>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  return hipGetLastError();
}

}  // namespace pxa
