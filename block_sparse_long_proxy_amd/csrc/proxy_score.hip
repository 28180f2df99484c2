// proxy_score.hip -- fused proxy QK^T + 128x128 block max-pool.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Score Estimation":
// token-level scores of the proxy head are max-pooled into block importance
// scores, with the QK product and the max pooling fused at block level.
// Causal prefill: in the diagonal block only keys j <= i count; blocks above
// the diagonal get -inf.
//
// The proxies come block-scaled (fp16 values times 2^e per proxy and 128-token
// block, e stored beside them): the fp16 MFMA products of tile (I, J) are the
// logits times 2^(e_I + e_J), so the tile max is multiplied by the exact
// factor 2^-(e_I + e_J) (and the softmax scale) when it is stored.
//
// A partial last block (128 does not divide N) is read with its missing rows
// replaced by copies of token N-1: every pair such a copy forms is a causal
// pair of token N-1, so its block maxima are those of the tokens present.
//
// With a query stride s (the sequence-level skip of section 5, read as
// scoring every s-th query of a block: offsets s-1, 2s-1, ..., 127) a
// workgroup serves s consecutive rows, 128/s queries each, so the per-tile
// work and the reuse of each K tile stay those of s = 1.
//
// One workgroup of four waves per proxy g and query-block row I (or, when
// few long rows would leave the chip idle, per 64-tile multiple of a row's
// key range: the chunks write disjoint score entries, so nothing is merged),
// two workgroups per CU (they run out of phase, so one's maxima and barriers
// overlap the other's MFMAs).  Key tiles J = 0..I stream through a two-deep
// LDS ring filled by direct global->LDS copies (tile J+1 lands while J is
// used).  Each wave computes 32 keys of the tile against all 128 proxy queries
// of the row, which stay in registers as MFMA B operands, so every K fragment
// read from LDS feeds four MFMAs; the fragment of the next k-step is read
// while the current one multiplies.  The max is taken in registers, across the
// wave with DPP moves (no LDS round trips), and kept in lane J mod 64; every
// 64 tiles the four waves combine their maxima through LDS and store them as
// one coalesced run, so the only per-tile barrier is the one guarding the ring.
#include <type_traits>

#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kScoreBufs = 2;                  // K tile in use + the next one in flight
// Wave priorities (s_setprio): a wave taking its block maxima (a short
// dependent VALU chain before the next barrier) issues ahead of the other
// workgroup's wave on the same SIMD, whose products fill in behind.
constexpr int kPrioProducts = 0;
constexpr int kPrioMax = 1;

// STRIDE s: the block's queries at offsets s-1, 2s-1, ..., 127 are scored
// (128/s of them, in QC = 4/s chunks of 32); s = 1 scores every query.
// SPLIT: workgroups cover W-tile parts of the rows (template parameter so the
// whole-row launches carry none of that index arithmetic).
template <int D, int STRIDE, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void proxy_score_kernel(
    const _Float16* __restrict__ qbar, const _Float16* __restrict__ kbar,
    const int32_t* __restrict__ qexp, const int32_t* __restrict__ kexp, float* __restrict__ scores,
    int G, float scale, int W, const SeqTable t) {
  // STRIDE s: rows I0, I0-1, ..., I0-s+1 share the workgroup, each with its
  // 128/s scored queries (offsets s-1, 2s-1, ..., 127), so every wave still
  // holds 4 chunks of 32 queries and each K tile feeds the same MFMA work.
  constexpr int R = STRIDE;          // rows per workgroup
  constexpr int QC = 4 / STRIDE;     // 32-query chunks per row
  static_assert(QC * STRIDE == 4, "stride 1, 2 or 4");
  __shared__ __attribute__((aligned(16))) _Float16 kt[kScoreBufs][kBlock * D];
  __shared__ float wm[2][R][kWaves][64];         // per-wave maxima of one 64-tile chunk

  // sequence of a fused batch (its workgroups are consecutive), then this
  // sequence's proxies and score grid
  const int sid = t.n == 1 ? 0 : seq_find(t.swg, t.n, (int)blockIdx.x);
  int bl = (int)blockIdx.x - t.swg[sid];
  const int N = t.tok[sid + 1] - t.tok[sid];
  qbar += (size_t)t.tok[sid] * G * D;
  kbar += (size_t)t.tok[sid] * G * D;
  scores += (size_t)G * t.sq[sid];
  const int nb = t.blk[sid + 1] - t.blk[sid];
  qexp += (size_t)G * t.blk[sid];
  kexp += (size_t)G * t.blk[sid];
  const int tail = N - (nb - 1) * kBlock;        // tokens of the last block (128 unless partial)
  // Level lev of a row group covers its key tiles [lev W, lev W + W); the
  // row groups that reach level lev are the ceil((nb - lev W) / R) longest
  // ones.  W >= nb: one level, a workgroup per row group.
  int lev = 0;
  if (SPLIT) {
    for (;;) {
      const int n_lev = G * ((nb - lev * W + R - 1) / R);
      if (bl < n_lev) break;
      bl -= n_lev;
      ++lev;
    }
  }
  const int g = bl % G;
  const int I0 = nb - 1 - R * (bl / G);          // top row; longest rows first
  const int J0 = SPLIT ? lev * W : 0;            // this workgroup's key tiles J0 .. J1
  const int J1 = SPLIT ? min(I0, J0 + W - 1) : I0;
  const int ws = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // keys 32 ws ..
  const int l = threadIdx.x & 63;
  const int hi = l >> 5;
  constexpr size_t kTile = (size_t)kBlock * D;

  // chunk c serves row I0 - c / QC; the lane's query offset inside that block
  auto qoff = [&](int c) { return STRIDE * (32 * (c % QC) + (l & 31)) + STRIDE - 1; };
  f16x8 qf[4][D / 16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int Ir = I0 - c / QC;
    if (Ir >= 0) {
      // past the end of a partial last block: a copy of token N-1, whose pairs
      // with the (equally clamped) keys are all causal pairs of token N-1, so
      // the block maxima are unchanged
      const int qt = min(Ir * kBlock + qoff(c), N - 1);
      load_qfrag<D>(qbar + ((size_t)g * N + (size_t)qt) * D, qf[c]);
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[c][s] = f16x8{};
    }
  }
  const _Float16* kb = uniform_ptr(kbar + (size_t)g * N * D);
  if (lev == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int Ir = I0 - r;
      if (Ir < 0) continue;
      float* srow = scores + ((size_t)g * nb + Ir) * nb;
      for (int J = Ir + 1 + threadIdx.x; J < nb; J += kThreads) srow[J] = -INFINITY;
    }
  }
  // Threads 0..64R-1: combine chunk cc (tiles 64cc .. 64cc+63) of the four
  // key slices, for row I0 - (thread / 64), and undo the block scales.
  auto store_chunk = [&](int cc) {
    if (threadIdx.x < 64 * R) {
      const int r = threadIdx.x >> 6;
      const int Ir = I0 - r;
      const int J = 64 * cc + l;
      if (Ir >= 0 && J <= Ir) {
        const float* p = &wm[cc & 1][r][0][l];
        const int ex = qexp[(size_t)g * nb + Ir] + kexp[(size_t)g * nb + J];
        scores[((size_t)g * nb + Ir) * nb + J] =
            ldexpf(fmaxf(fmaxf(p[0], p[64]), fmaxf(p[128], p[192])), -ex) * scale;
      }
    }
  };

  // key tile J into buffer b; only tile nb-1 can be partial
  auto load_tile = [&](int J, _Float16* buf) {
    if (J == nb - 1 && tail < kBlock)
      tile_load_lds_rows<D, false>(kb + (size_t)J * kTile, buf, tail);
    else
      tile_load_lds<D, false>(kb + (size_t)J * kTile, buf);
  };
  load_tile(J0, kt[J0 % kScoreBufs]);
  float keep[R];                                 // this wave's max of tile J per row, lane J mod 64
#pragma unroll
  for (int r = 0; r < R; ++r) keep[r] = -INFINITY;
  for (int J = J0; J <= J1; ++J) {
    wait_vmem();       // this thread's part of tile J (the only copy in flight)
    __syncthreads();   // tile J visible; tile J-1's buffer is no longer read
    if (J + 1 <= J1) load_tile(J + 1, kt[(J + 1) % kScoreBufs]);
    if (J > J0 && (J & 63) == 0) store_chunk((J >> 6) - 1);   // written before the barrier
    const _Float16* cur = kt[J % kScoreBufs];
    f32x16 acc[4];
    __builtin_amdgcn_s_setprio(kPrioProducts);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = zero16();
    // The fragment of k-step s+1 is read before the four products of step s
    // issue (scheduling barriers keep that order; the default schedule reuses
    // one register set and waits for every read).
    f16x8 a = ktile_frag<D>(cur, ws, 0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      f16x8 an = a;
      if (s + 1 < D / 16) an = ktile_frag<D>(cur, ws, s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, qf[c][s], acc[c]);
      __builtin_amdgcn_sched_barrier(0);
      a = an;
    }
    __builtin_amdgcn_s_setprio(kPrioMax);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int Ir = I0 - r;
      float mx = -INFINITY;
      if (J < Ir) {
#pragma unroll
        for (int cc = 0; cc < QC; ++cc)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[r * QC + cc][e]);
      } else if (J == Ir) {   // causal: key 32 ws + row(e) must not exceed the lane's query
#pragma unroll
        for (int cc = 0; cc < QC; ++cc)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 32 * ws + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (key <= qoff(r * QC + cc)) mx = fmaxf(mx, acc[r * QC + cc][e]);
          }
      }                       // J > Ir: above that row's diagonal, nothing counts
      mx = wave_max_uniform(mx);
      if (l == (J & 63)) keep[r] = mx;
    }
    if ((J & 63) == 63 || J == J1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wm[(J >> 6) & 1][r][ws][l] = keep[r];
        keep[r] = -INFINITY;
      }
    }
  }
  // J1 ends a 64-tile chunk or is I0, so every entry stored was computed here
  __syncthreads();
  store_chunk(J1 >> 6);
}

// Workgroup slots of the chip for this kernel (256 CUs, two workgroups each).
constexpr long kScoreSlots = 512;

hipError_t launch_proxy_score(const LaunchArgs& a, const SeqTable& t, const void* qbar,
                              const void* kbar, const int32_t* qexp, const int32_t* kexp,
                              float* scores, hipStream_t stream) {
  // Key tiles per workgroup: whole rows when the longest row is at most half
  // the mean load of a slot (the longest-first order then balances), else
  // multiples of 64 tiles near that half, so a few long rows do not leave
  // most of the chip idle.
  const int R = a.score_stride;
  long tiles = 0;
  int nbmax = 0;
  for (int s = 0; s < t.n; ++s) {
    const int nb = t.blk[s + 1] - t.blk[s];
    nbmax = nb > nbmax ? nb : nbmax;
    for (int top = nb; top > 0; top -= R) tiles += (long)a.G * top;   // row group: top tiles
  }
  const long half_mean = tiles / kScoreSlots / 2;
  int W = (int)align_up((size_t)nbmax, 64);
  if (nbmax > half_mean) W = (int)(half_mean / 64 > 1 ? half_mean / 64 * 64 : 64);
  SeqTable tw = t;   // workgroup prefix for this chunking
  tw.swg[0] = 0;
  for (int s = 0; s < t.n; ++s) {
    const int nb = t.blk[s + 1] - t.blk[s];
    int wgs = 0;
    for (int lev = 0; nb - lev * W > 0; ++lev) wgs += a.G * ((nb - lev * W + R - 1) / R);
    tw.swg[s + 1] = tw.swg[s] + wgs;
  }
  const dim3 grid(tw.swg[t.n]), block(kThreads);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, (const _Float16*)qbar,
                       (const _Float16*)kbar, qexp, kexp, scores, a.G, a.scale, W, tw);
  };
  const bool split = W < nbmax;
  auto pick = [&](auto d) {
    constexpr int D = decltype(d)::value;
    if (split) {
      if (a.score_stride == 4) go(proxy_score_kernel<D, 4, true>);
      else if (a.score_stride == 2) go(proxy_score_kernel<D, 2, true>);
      else go(proxy_score_kernel<D, 1, true>);
    } else {
      if (a.score_stride == 4) go(proxy_score_kernel<D, 4, false>);
      else if (a.score_stride == 2) go(proxy_score_kernel<D, 2, false>);
      else go(proxy_score_kernel<D, 1, false>);
    }
  };
  if (a.D == 64) pick(std::integral_constant<int, 64>{});
  else pick(std::integral_constant<int, 128>{});
  return hipGetLastError();
}

}  // namespace pxa
