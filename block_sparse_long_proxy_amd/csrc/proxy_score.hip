// proxy_score.hip -- fused proxy QK^T + 128x128 block max-pool.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Score Estimation":
// token-level scores of the proxy head are max-pooled into block importance
// scores, with the QK product and the max pooling fused at block level.
// Causal prefill: in the diagonal block only keys j <= i count; blocks above
// the diagonal get -inf.
//
// One workgroup per proxy g and pair of query-block rows (I, I-1).  Key tiles
// J = 0..I stream through a three-deep LDS ring filled by direct global->LDS
// copies (tiles J+1 and J+2 are in flight while J is used).  Each of the eight
// waves computes 32 keys of the tile against all 128 proxy queries of its row,
// which stay in registers as MFMA B operands, so every K fragment read from
// LDS feeds four MFMAs.  The max is taken in registers, across the wave with
// DPP moves (no LDS round trips), and kept in lane J mod 64; every 64 tiles the
// four waves of a row combine their maxima through LDS and store them as one
// coalesced run, so the only per-tile barrier is the one guarding the ring.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kScoreWaves = 8;                 // two rows x four key slices
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kScoreBufs = 3;                  // K tiles in flight / in use

// Direct global->LDS copy of one [128][D] K tile by all kScoreThreads threads
// (the tile_load_lds scheme with eight waves).
template <int D>
__device__ __forceinline__ void score_tile_load(const __bf16* __restrict__ g, __bf16* lds) {
  constexpr int C = D / 8;
  constexpr int ROWS = 64 / C;
  constexpr int INSTS = kBlock / ROWS / kScoreWaves;
  static_assert((kScoreWaves * ROWS) % 16 == 0, "swizzle must repeat every instruction");
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  g = uniform_ptr(g);
  const int row0 = w * ROWS + l / C;
  const int logical = (l % C) ^ kswz<D>(row0);
  const uint32_t voff = (uint32_t)((l / C) * D + logical * 8) * 2u;
  const uint32_t lbase = lds_addr(lds) + (uint32_t)(w * ROWS * D * 2);
#pragma unroll
  for (int it = 0; it < INSTS; ++it) {
    const int blk_row = (it * kScoreWaves + w) * ROWS;
    lds_dma16(g + (size_t)blk_row * D, voff, lbase + (uint32_t)(it * kScoreWaves * ROWS * D * 2));
  }
}

// Waves 0-3 serve row I, waves 4-7 row I-1 (absent when I == 0).  Both rows
// need key tiles 0..I-1, so each staged tile feeds twice the MFMA work.  The
// block maximum of tile J stays in lane J mod 64 of each wave; every 64 tiles
// the four slices of a row are combined through LDS and stored as one
// coalesced run of scores.
template <int D>
__global__ __launch_bounds__(kScoreThreads, 1) void proxy_score_kernel(
    const __bf16* __restrict__ qbar, const __bf16* __restrict__ kbar, float* __restrict__ scores,
    int G, int N, float scale) {
  __shared__ __attribute__((aligned(16))) __bf16 kt[kScoreBufs][kBlock * D];
  __shared__ float wm[2][kScoreWaves][64];       // per-wave maxima of one 64-tile chunk

  const int nb = N / kBlock;
  const int pair = (int)(blockIdx.x / G);        // longest rows first
  const int g = (int)(blockIdx.x % G);
  const int I = nb - 1 - 2 * pair;               // top row of the pair
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = threadIdx.x & 63;
  const int rsel = w >> 2;                       // 0: row I, 1: row I-1
  const int ws = w & 3;                          // key slice 32 ws .. 32 ws + 31
  const int myI = I - rsel;
  const bool active = myI >= 0;
  constexpr size_t kTile = (size_t)kBlock * D;
  constexpr int kLoadsPerTile = kBlock / (64 / (D / 8)) / kScoreWaves;

  bf16x8 qf[4][D / 16];
  if (active) {
#pragma unroll
    for (int qs = 0; qs < 4; ++qs)
      load_qfrag<D>(qbar + ((size_t)g * N + (size_t)myI * kBlock + 32 * qs + (l & 31)) * D, qf[qs]);
  }
  const __bf16* kb = uniform_ptr(kbar + (size_t)g * N * D);
  float* srow0 = scores + ((size_t)g * nb + I) * nb;
  for (int J = I + 1 + threadIdx.x; J < nb; J += kScoreThreads) srow0[J] = -INFINITY;
  if (I >= 1) {
    float* srow1 = srow0 - nb;
    for (int J = I + threadIdx.x; J < nb; J += kScoreThreads) srow1[J] = -INFINITY;
  }
  // Threads 0..127: combine chunk c (tiles 64c .. 64c+63) of rows I and I-1.
  auto store_chunk = [&](int c) {
    if (threadIdx.x < 128) {
      const int rr = threadIdx.x >> 6;
      const int J = 64 * c + l;
      if (J <= I - rr) {
        const float* p = &wm[c & 1][4 * rr][l];
        srow0[J - (size_t)rr * nb] = fmaxf(fmaxf(p[0], p[64]), fmaxf(p[128], p[192])) * scale;
      }
    }
  };

  // prologue: tiles 0 .. kScoreBufs-2 in flight
#pragma unroll
  for (int p = 0; p < kScoreBufs - 1; ++p)
    if (p <= I) score_tile_load<D>(kb + (size_t)p * kTile, kt[p]);
  const int hi = l >> 5;
  float keep = -INFINITY;                        // this wave's max of tile J, in lane J mod 64
  for (int J = 0; J <= I; ++J) {
    // wait for this thread's part of tile J; tile J+1 may stay in flight
    if (J + 1 <= I)
      wait_vmem_le<kLoadsPerTile>();
    else
      wait_vmem();
    __syncthreads();   // tile J visible; tile J-1's buffer is no longer read
    if (J + kScoreBufs - 1 <= I)
      score_tile_load<D>(kb + (size_t)(J + kScoreBufs - 1) * kTile,
                         kt[(J + kScoreBufs - 1) % kScoreBufs]);
    if (J > 0 && (J & 63) == 0) store_chunk((J >> 6) - 1);   // written before the barrier
    float mx = -INFINITY;
    if (active && J <= myI) {
      const __bf16* cur = kt[J % kScoreBufs];
      f32x16 acc[4];
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) acc[qs] = zero16();
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 a = ktile_frag<D>(cur, ws, s);
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) acc[qs] = mfma32(a, qf[qs][s], acc[qs]);
      }
      if (J == myI) {   // causal: key 32 ws + row(r) must not exceed query 32 qs + l%32
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
    }
    if (l == (J & 63)) keep = mx;
    if ((J & 63) == 63 || J == I) {
      wm[(J >> 6) & 1][w][l] = keep;
      keep = -INFINITY;
    }
  }
  __syncthreads();
  store_chunk(I >> 6);
}

hipError_t launch_proxy_score(const LaunchArgs& a, const void* qbar, const void* kbar,
                              float* scores, hipStream_t stream) {
  const int nb = a.N / kBlock;
  const dim3 grid(a.G * ((nb + 1) / 2)), block(kScoreThreads);
  if (a.D == 64)
    hipLaunchKernelGGL(proxy_score_kernel<64>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  else
    hipLaunchKernelGGL(proxy_score_kernel<128>, grid, block, 0, stream, (const __bf16*)qbar,
                       (const __bf16*)kbar, scores, a.G, a.N, a.scale);
  return hipGetLastError();
}

}  // namespace pxa
