// proxy_pool.hip -- head pooling into proxy heads.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Head Pooling": Q and
// K of the heads in one group are aggregated over the head dimension into a
// proxy head (section 3 describes it as a simple pooling).  Reading: the mean.
// qbar[g] = mean of q over query heads [g*H/G, (g+1)*H/G); kbar[g] = mean of
// k over the contiguous KV heads those query heads use.
//
// Pure streaming: every thread owns one 16-byte chunk (8 dims of one token)
// of one proxy, sums the member heads' chunks in fp32 in head order, divides
// by the member count and rounds once to bf16.  Grid z covers (sequence,
// Q or K) of a fused batch; each sequence's tensors start after the previous
// ones.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

__global__ __launch_bounds__(256) void proxy_pool_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, __bf16* __restrict__ qbar,
    __bf16* __restrict__ kbar, int H, int Hkv, int G, int D, const SeqTable t) {
  const int s = (int)(blockIdx.z >> 1);        // sequence
  const bool is_k = (blockIdx.z & 1) != 0;
  const size_t tok0 = (size_t)t.tok[s];
  const size_t head_elems = (size_t)(t.tok[s + 1] - t.tok[s]) * D;
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= head_elems / 8) return;
  const int g = blockIdx.y;
  const int qpg = H / G;                       // query heads per group
  int first, count;
  if (!is_k) {
    first = g * qpg;
    count = qpg;
  } else {
    const int qpk = H / Hkv;                   // query heads per KV head
    first = (g * qpg) / qpk;
    count = ((g + 1) * qpg - 1) / qpk - first + 1;
  }
  const __bf16* src = (is_k ? k + tok0 * Hkv * D : q + tok0 * H * D) +
                      (size_t)first * head_elems + c * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // member heads in order, their loads issued four at a time
  int i = 0;
  for (; i + 4 <= count; i += 4) {
    bf16x8 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const bf16x8*>(src + (size_t)(i + u) * head_elems);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)x[u][e];
  }
  for (; i < count; ++i) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(src + (size_t)i * head_elems);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
  }
  const float n = (float)count;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] / n);
  __bf16* dst = (is_k ? kbar : qbar) + tok0 * G * D + (size_t)g * head_elems + c * 8;
  *reinterpret_cast<bf16x8*>(dst) = out;
}

hipError_t launch_proxy_pool(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                             void* qbar, void* kbar, hipStream_t stream) {
  const size_t chunks = (size_t)max_len(t) * a.D / 8;   // of the longest sequence
  const dim3 grid((unsigned)((chunks + 255) / 256), a.G, 2 * t.n), block(256);
  hipLaunchKernelGGL(proxy_pool_kernel, grid, block, 0, stream, (const __bf16*)q,
                     (const __bf16*)k, (__bf16*)qbar, (__bf16*)kbar, a.H, a.Hkv, a.G, a.D, t);
  return hipGetLastError();
}

}  // namespace pxa
