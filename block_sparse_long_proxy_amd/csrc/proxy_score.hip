// proxy_score.hip -- fused proxy QK^T + 128x128 block max-pool.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Score Estimation":
// token-level scores of the proxy head are max-pooled into block importance
// scores, with the QK product and the max pooling fused at block level.
// Causal prefill: in the diagonal block only keys j <= i count; blocks above
// the diagonal get -inf.
//
// One workgroup of four waves per proxy g and query-block row I, two
// workgroups per CU (they run out of phase, so one's maxima and barriers
// overlap the other's MFMAs).  Key tiles J = 0..I stream through a two-deep
// LDS ring filled by direct global->LDS copies (tile J+1 lands while J is
// used).  Each wave computes 32 keys of the tile against all 128 proxy queries
// of the row, which stay in registers as MFMA B operands, so every K fragment
// read from LDS feeds four MFMAs; the fragment of the next k-step is read
// while the current one multiplies.  The max is taken in registers, across the
// wave with DPP moves (no LDS round trips), and kept in lane J mod 64; every
// 64 tiles the four waves combine their maxima through LDS and store them as
// one coalesced run, so the only per-tile barrier is the one guarding the ring.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kScoreBufs = 2;                  // K tile in use + the next one in flight

template <int D>
__global__ __launch_bounds__(kThreads, 2) void proxy_score_kernel(
    const __bf16* __restrict__ qbar, const __bf16* __restrict__ kbar, float* __restrict__ scores,
    int G, int N, float scale) {
  __shared__ __attribute__((aligned(16))) __bf16 kt[kScoreBufs][kBlock * D];
  __shared__ float wm[2][kWaves][64];            // per-wave maxima of one 64-tile chunk

  const int nb = N / kBlock;
  const int g = (int)(blockIdx.x % G);
  const int I = nb - 1 - (int)(blockIdx.x / G);  // longest rows first
  const int ws = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // keys 32 ws ..
  const int l = threadIdx.x & 63;
  const int hi = l >> 5;
  constexpr size_t kTile = (size_t)kBlock * D;

  bf16x8 qf[4][D / 16];
#pragma unroll
  for (int qs = 0; qs < 4; ++qs)
    load_qfrag<D>(qbar + ((size_t)g * N + (size_t)I * kBlock + 32 * qs + (l & 31)) * D, qf[qs]);
  const __bf16* kb = uniform_ptr(kbar + (size_t)g * N * D);
  float* srow = scores + ((size_t)g * nb + I) * nb;
  for (int J = I + 1 + threadIdx.x; J < nb; J += kThreads) srow[J] = -INFINITY;
  // Wave 0: combine chunk c (tiles 64c .. 64c+63) of the four slices.
  auto store_chunk = [&](int c) {
    if (threadIdx.x < 64) {
      const int J = 64 * c + l;
      if (J <= I) {
        const float* p = &wm[c & 1][0][l];
        srow[J] = fmaxf(fmaxf(p[0], p[64]), fmaxf(p[128], p[192])) * scale;
      }
    }
  };

  tile_load_lds<D, false>(kb, kt[0]);
  float keep = -INFINITY;                        // this wave's max of tile J, in lane J mod 64
  for (int J = 0; J <= I; ++J) {
    wait_vmem();       // this thread's part of tile J (the only copy in flight)
    __syncthreads();   // tile J visible; tile J-1's buffer is no longer read
    if (J + 1 <= I) tile_load_lds<D, false>(kb + (size_t)(J + 1) * kTile, kt[(J + 1) % kScoreBufs]);
    if (J > 0 && (J & 63) == 0) store_chunk((J >> 6) - 1);   // written before the barrier
    const __bf16* cur = kt[J % kScoreBufs];
    f32x16 acc[4];
#pragma unroll
    for (int qs = 0; qs < 4; ++qs) acc[qs] = zero16();
    // The fragment of k-step s+1 is read before the four products of step s
    // issue (scheduling barriers keep that order; the default schedule reuses
    // one register set and waits for every read).
    bf16x8 a = ktile_frag<D>(cur, ws, 0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 an = a;
      if (s + 1 < D / 16) an = ktile_frag<D>(cur, ws, s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) acc[qs] = mfma32(a, qf[qs][s], acc[qs]);
      __builtin_amdgcn_sched_barrier(0);
      a = an;
    }
    float mx = -INFINITY;
    if (J == I) {   // causal: key 32 ws + row(r) must not exceed query 32 qs + l%32
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * ws + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key <= 32 * qs + (l & 31)) mx = fmaxf(mx, acc[qs][r]);
        }
    } else {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[qs][r]);
    }
    mx = wave_max_uniform(mx);
    if (l == (J & 63)) keep = mx;
    if ((J & 63) == 63 || J == I) {
      wm[(J >> 6) & 1][ws][l] = keep;
      keep = -INFINITY;
    }
  }
  __syncthreads();
  store_chunk(I >> 6);
}

hipError_t launch_proxy_score(const LaunchArgs& a, const void* qbar, const void* kbar,
                              float* scores, hipStream_t stream) {
  const int nb = a.N / kBlock;
  const dim3 grid(a.G * nb), block(kThreads);
  if (a.D == 64)
    hipLaunchKernelGGL(proxy_score_kernel<64>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  else
    hipLaunchKernelGGL(proxy_score_kernel<128>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  return hipGetLastError();
}

}  // namespace pxa
