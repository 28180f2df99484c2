// proxy_pool.hip -- head pooling into proxy heads.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Head Pooling": Q and
// K of the heads in one group are aggregated over the head dimension into a
// proxy head (section 3 describes it as a simple pooling).  Reading: the mean.
// qbar[g] = mean of q over query heads [g*H/G, (g+1)*H/G); kbar[g] = mean of
// k over the contiguous KV heads those query heads use.
//
// Storage: block-scaled fp16.  Each (proxy, 128-token block) gets a power of
// two 2^e chosen so that the block's largest |mean| lands in [2^14, 2^15);
// the proxy holds fp16(mean * 2^e) (round to nearest even) and e is stored
// beside it.  Every element keeps 11 significant bits (8 in bf16), no finite
// input can overflow, and a block score only needs the exact factor
// 2^-(e_I + e_J) applied to the max of its tile.
//
// One workgroup of 256 threads per (sequence, proxy, block, Q or K): a thread
// owns 8 (d = 128) or 4 (d = 64) 16-byte chunks of the block, sums the member
// heads' chunks in fp32 in head order, divides by the member count (IEEE
// division), and the workgroup reduces the block's largest |mean| before the
// scaled values are rounded and stored.  Rows past the end of a partial last
// block are neither read nor written.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kPoolThreads = 256;

template <int D>
__global__ __launch_bounds__(kPoolThreads) void proxy_pool_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, _Float16* __restrict__ qbar,
    _Float16* __restrict__ kbar, int32_t* __restrict__ qexp, int32_t* __restrict__ kexp, int H,
    int Hkv, int G, const SeqTable t) {
  constexpr int C = D / 8;                           // 16-byte chunks per token
  constexpr int PER = kBlock * C / kPoolThreads;     // chunks per thread
  __shared__ float wmax[kPoolThreads / 64];
  const int s = (int)(blockIdx.z >> 1);              // sequence
  const bool is_k = (blockIdx.z & 1) != 0;
  const int nb = t.blk[s + 1] - t.blk[s];
  const int I = blockIdx.x;
  if (I >= nb) return;                               // the grid covers the longest sequence
  const int N = t.tok[s + 1] - t.tok[s];
  const int rows = min(kBlock, N - I * kBlock);      // tokens of this block
  const int g = blockIdx.y;
  const int qpg = H / G;                             // query heads per group
  int first, count;
  if (!is_k) {
    first = g * qpg;
    count = qpg;
  } else {
    const int qpk = H / Hkv;                         // query heads per KV head
    first = (g * qpg) / qpk;
    count = ((g + 1) * qpg - 1) / qpk - first + 1;
  }
  const size_t tok0 = (size_t)t.tok[s];
  const size_t head_elems = (size_t)N * D;
  const __bf16* src = (is_k ? k + tok0 * Hkv * D : q + tok0 * H * D) +
                      (size_t)first * head_elems + (size_t)I * kBlock * D;
  const int tid = threadIdx.x;

  // chunk p of this thread: element offset off[p] inside the block; a chunk
  // of a row past a partial block's end re-reads the last row (never stored)
  int off[PER];
  bool valid[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = p * kPoolThreads + tid;
    const int row = c / C;
    valid[p] = row < rows;
    off[p] = (valid[p] ? row : rows - 1) * D + (c % C) * 8;
  }
  float acc[PER][8];
#pragma unroll
  for (int p = 0; p < PER; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[p][e] = 0.f;
  for (int i = 0; i < count; ++i) {                  // member heads in order
    const __bf16* h = src + (size_t)i * head_elems;
    bf16x8 x[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) x[p] = *reinterpret_cast<const bf16x8*>(h + off[p]);
#pragma unroll
    for (int p = 0; p < PER; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[p][e] += (float)x[p][e];
  }
  const float n = (float)count;
  float mx = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[p][e] = acc[p][e] / n;
      if (valid[p]) mx = fmaxf(mx, fabsf(acc[p][e]));
    }
  mx = wave_max_uniform(mx);
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kPoolThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);
  // mx = f 2^x with f in [0.5, 1): mx 2^(15 - x) = f 2^15 lies in [2^14, 2^15)
  int ex = 0;
  if (mx > 0.f) {
    int x;
    frexpf(mx, &x);
    ex = 15 - x;
  }
  _Float16* dst = (is_k ? kbar : qbar) + tok0 * G * D + (size_t)g * head_elems +
                  (size_t)I * kBlock * D;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    if (!valid[p]) continue;
    f16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (_Float16)ldexpf(acc[p][e], ex);
    *reinterpret_cast<f16x8*>(dst + off[p]) = out;
  }
  if (tid == 0) (is_k ? kexp : qexp)[(size_t)G * t.blk[s] + (size_t)g * nb + I] = ex;
}

hipError_t launch_proxy_pool(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                             void* qbar, void* kbar, int32_t* qexp, int32_t* kexp,
                             hipStream_t stream) {
  const dim3 grid((unsigned)max_blocks(t), a.G, 2 * t.n), block(kPoolThreads);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (_Float16*)qbar, (_Float16*)kbar, qexp, kexp, a.H, a.Hkv, a.G, t);
  };
  if (a.D == 64) go(proxy_pool_kernel<64>);
  else go(proxy_pool_kernel<128>);
  return hipGetLastError();
}

}  // namespace pxa
