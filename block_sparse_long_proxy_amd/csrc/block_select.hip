// block_select.hip -- block ranking + per-head top-k -> CSR block mask.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, step 1 "Block Ranking": the
// key blocks of each row are ranked by the proxy block scores and the top
// blocks within a budget are kept; the final step combines that ranking with
// the per-head budgets of step 2 into the block sparse mask.  Row (h, I)
// keeps the first min(k_h, I+1) blocks of its group's ranking (score
// descending, block ascending on ties) plus the diagonal block I.
//
// Three launches:
//   select_count_kernel: one wave per (g, I); the rank of the diagonal block
//     is a plain count of blocks ahead of it, so the row lengths (and hence
//     row_ptr) are known without sorting.
//   select_scan_kernel : exclusive scan of the H*nb lengths -> row_ptr, and
//     the XCD-aware, longest-first schedule of the rows -> row_order.
// A fused batch has one CSR over the rows of all its sequences (sequence s's
// rows follow those of the sequences before it), so the scan and the
// schedule balance the XCDs over the whole batch.
//   select_emit_kernel : one workgroup per (g, I); bitonic sort of the row's
//     64-bit (score, index) keys in LDS gives every block's rank; each head
//     of the group then compacts {J : rank < k or J == I} in ascending J.
#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

constexpr int kEmitThreads = 256;
constexpr int kScanThreads = 1024;

// Ranked blocks row I keeps under the ratio budget r: ceil of the float32
// product r * (I+1) (nearest-even, no contraction), within [1, I+1].  (The
// Top-K-by-proportion choice of the XAttention report, section 2.2.)
__device__ __forceinline__ int ratio_count(int I, float r) {
  const float prod = __fmul_rn(r, (float)(I + 1));
  return min(I + 1, max(1, (int)ceilf(prod)));
}

// Budget of row I in head h: the head's k_h, or the ratio budget when k_h is NULL.
__device__ __forceinline__ int row_budget(const int32_t* __restrict__ k_h, int h, int I,
                                          float ratio) {
  return k_h ? max(0, min(k_h[h], I + 1)) : ratio_count(I, ratio);
}

__global__ __launch_bounds__(256) void select_count_kernel(const float* __restrict__ scores,
                                                           const int32_t* __restrict__ k_h,
                                                           int32_t* __restrict__ counts, int H,
                                                           int G, float ratio, const SeqTable t) {
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);   // G * blk[sid] + g * nb + I
  const int l = threadIdx.x & 63;
  if (gr >= G * t.blk[t.n]) return;
  const int sid = t.n == 1 ? 0 : seq_find(t.blk, t.n, gr / G);
  const int nb = t.blk[sid + 1] - t.blk[sid];
  const int row = gr - G * t.blk[sid];                 // g * nb + I in this sequence
  const int g = row / nb, I = row % nb;
  counts += (size_t)H * t.blk[sid];
  if (k_h) k_h += (size_t)H * sid;
  const float* s = scores + (size_t)G * t.sq[sid] + (size_t)row * nb;
  const uint64_t kd = rank_key(s[I], (uint32_t)I);
  int ahead = 0;
  for (int J = l; J < I; J += 64) ahead += rank_key(s[J], (uint32_t)J) < kd ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ahead += __shfl_xor(ahead, o, 64);
  const int hpg = H / G;
  for (int hh = l; hh < hpg; hh += 64) {
    const int h = g * hpg + hh;
    const int kk = row_budget(k_h, h, I, ratio);   // negative budgets: diagonal only
    counts[(size_t)h * nb + I] = kk + (ahead >= kk ? 1 : 0);
  }
}

// Exclusive scan of the n row lengths into row_ptr[0..n]; optionally also the
// attention kernel's schedule row_order.  Workgroup b of a launch goes to XCD
// b mod 8, and each XCD has its own L2, so the schedule is built per XCD:
//   * XCD x owns the rows whose midpoint in the cumulative work row_ptr falls
//     in the x-th eighth.  Rows are numbered h * nb + I and the heads of one
//     KV head are consecutive, so each XCD sees one or two KV heads and their
//     K/V tiles stay in its L2;
//   * position p of row_order is dealt to XCD p mod 8, so XCD x holds exactly
//     cap_x = ceil-or-floor(n / 8) positions; its own rows fill them longest
//     first, a surplus (its shortest rows) moves to XCDs with spare positions.
// The longest-first order P comes from a counting sort by length (rows of
// equal length in no fixed order) into tmp[n]; stable ranks along P per XCD
// come from a block-wide scan of eight counters.  One workgroup; hist needs
// max_len + 1 ints of dynamic LDS.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_of_row(int64_t start, int len, int64_t total) {
  // midpoint (start + len/2) scaled to [0, 8)
  const int64_t x = ((2 * start + len) * kXcds) / (2 * total);
  return (int)min<int64_t>(x, kXcds - 1);
}

// f(i, counts[i]) for i in [a, b) in order, the loads issued eight at a time
// (one at a time, these loops wait out a memory latency per row).
template <typename F>
__device__ __forceinline__ void for_counts(const int32_t* __restrict__ counts, int a, int b,
                                           F&& f) {
  int i = a;
  for (; i + 8 <= b; i += 8) {
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = counts[i + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) f(i + u, c[u]);
  }
  for (; i < b; ++i) f(i, counts[i]);
}

// f(r, counts[r], row_ptr[r]) for the rows r = tmp[p], p in [a, b), in order,
// with the loads batched the same way.
template <typename F>
__device__ __forceinline__ void for_order(const int32_t* __restrict__ tmp,
                                          const int32_t* __restrict__ counts,
                                          const int32_t* __restrict__ row_ptr, int a, int b,
                                          F&& f) {
  int p = a;
  for (; p + 8 <= b; p += 8) {
    int r[8], c[8], s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = tmp[p + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = counts[r[u]];
      s[u] = row_ptr[r[u]];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) f(r[u], c[u], s[u]);
  }
  for (; p < b; ++p) {
    const int r = tmp[p];
    f(r, counts[r], row_ptr[r]);
  }
}

// Inclusive Hillis-Steele scan of part[0..kScanThreads) in place.
__device__ __forceinline__ void block_scan(int* part) {
  const int t = threadIdx.x;
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int x = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kScanThreads) void select_scan_kernel(const int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ row_ptr,
                                                                   int32_t* __restrict__ row_order,
                                                                   int32_t* __restrict__ tmp,
                                                                   int n, int max_len) {
  __shared__ int part[kScanThreads];
  __shared__ int xc[kScanThreads][kXcds];   // per-thread counts, then exclusive prefixes
  __shared__ int xtot[kXcds];
  extern __shared__ int hist[];   // [max_len + 1]
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int a = min(n, t * per), b = min(n, a + per);
  int s = 0;
  for_counts(counts, a, b, [&](int, int c) { s += c; });
  part[t] = s;
  if (row_order)
    for (int c = t; c <= max_len; c += kScanThreads) hist[c] = 0;
  __syncthreads();
  block_scan(part);
  int run = part[t] - s;
  for_counts(counts, a, b, [&](int i, int c) {
    row_ptr[i] = run;
    run += c;
  });
  if (t == kScanThreads - 1) row_ptr[n] = part[t];
  if (!row_order) return;
  const int64_t total = part[kScanThreads - 1];

  // P = rows longest first (counting sort)
  for_counts(counts, a, b, [&](int, int c) { atomicAdd(&hist[min(c, max_len)], 1); });
  __syncthreads();   // hist complete; every read of part above is done
  {   // bucket starts, longest bucket first: exclusive scan of hist taken from c = max_len down
    const int nbk = max_len + 1;
    const int per2 = (nbk + kScanThreads - 1) / kScanThreads;
    const int q0 = min(nbk, t * per2), q1 = min(nbk, q0 + per2);
    int sum = 0;
    for (int q = q0; q < q1; ++q) sum += hist[max_len - q];
    part[t] = sum;
    __syncthreads();
    block_scan(part);
    int acc = part[t] - sum;
    for (int q = q0; q < q1; ++q) {
      const int x = hist[max_len - q];
      hist[max_len - q] = acc;
      acc += x;
    }
  }
  __syncthreads();
  for_counts(counts, a, b, [&](int i, int c) { tmp[atomicAdd(&hist[min(c, max_len)], 1)] = i; });
  __syncthreads();   // tmp complete: the barrier's fence orders the global writes

  // per-XCD ranks along P: counts of this thread's positions [a, b) of P
  int mine[kXcds];
#pragma unroll
  for (int x = 0; x < kXcds; ++x) mine[x] = 0;
  for_order(tmp, counts, row_ptr, a, b,
            [&](int, int c, int start) { mine[xcd_of_row(start, c, total)]++; });
#pragma unroll
  for (int x = 0; x < kXcds; ++x) xc[t][x] = mine[x];
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {   // inclusive scan of 8 columns
    int add[kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x) add[x] = t >= off ? xc[t - off][x] : 0;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kXcds; ++x) xc[t][x] += add[x];
    __syncthreads();
  }
  if (t < kXcds) xtot[t] = xc[kScanThreads - 1][t];
  __syncthreads();
  int cnt[kXcds], cap[kXcds], deficit_start[kXcds + 1];
  deficit_start[0] = 0;
#pragma unroll
  for (int x = 0; x < kXcds; ++x) {
    cnt[x] = xc[t][x] - mine[x];                       // ranks before this segment
    cap[x] = n / kXcds + (x < n % kXcds ? 1 : 0);      // positions dealt to XCD x
    deficit_start[x + 1] = deficit_start[x] + max(0, cap[x] - xtot[x]);
  }
  for_order(tmp, counts, row_ptr, a, b, [&](int r, int c, int start) {
    const int x = xcd_of_row(start, c, total);
    int pos;
    if (cnt[x] < cap[x]) {
      pos = kXcds * cnt[x] + x;
    } else {   // surplus: the sj-th surplus row along P takes the sj-th spare position
      int sj = 0;
#pragma unroll
      for (int y = 0; y < kXcds; ++y) sj += max(0, cnt[y] - cap[y]);
      int y = 0;
      while (y < kXcds - 1 && sj >= deficit_start[y + 1]) ++y;
      pos = kXcds * (xtot[y] + (sj - deficit_start[y])) + y;
    }
    cnt[x]++;
    row_order[pos] = r;
  });
}

__global__ __launch_bounds__(kEmitThreads) void select_emit_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ k_h,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int H, int G,
    int Pmax, float ratio, const SeqTable st) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);          // [Pmax]
  uint16_t* rank = reinterpret_cast<uint16_t*>(keys + Pmax);   // [nb]
  __shared__ int wsum[kEmitThreads / 64];

  // Sequence of a fused batch; within it heavy rows first: (I descending, g).
  const int sid = st.n == 1 ? 0 : seq_find(st.blk, st.n, (int)blockIdx.x / G);
  const int bl = (int)blockIdx.x - G * st.blk[sid];
  const int nb = st.blk[sid + 1] - st.blk[sid];
  scores += (size_t)G * st.sq[sid];
  if (k_h) k_h += (size_t)H * sid;
  row_ptr += (size_t)H * st.blk[sid];       // this sequence's rows of the fused CSR
  const int I = nb - 1 - bl / G;
  const int g = bl % G;
  const int n = I + 1;
  int P = 1;
  while (P < n) P <<= 1;
  const int t = threadIdx.x;
  const float* s = scores + ((size_t)g * nb + I) * nb;
  for (int J = t; J < P; J += kEmitThreads)
    keys[J] = J < n ? rank_key(s[J], (uint32_t)J) : ~0ull;
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P / 2; i += kEmitThreads) {
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
  for (int r = t; r < n; r += kEmitThreads) rank[(uint32_t)keys[r]] = (uint16_t)r;
  __syncthreads();

  // Contiguous chunk of J per thread so the output stays in ascending order.
  const int per = (n + kEmitThreads - 1) / kEmitThreads;
  const int a0 = min(n, t * per), a1 = min(n, a0 + per);
  const int hpg = H / G;
  const int wv = t >> 6, ln = t & 63;
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int kk = row_budget(k_h, h, I, ratio);
    int c = 0;
    for (int J = a0; J < a1; ++J) c += (rank[J] < kk || J == I) ? 1 : 0;
    // exclusive scan of c over the workgroup
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (ln >= o) incl += y;
    }
    if (ln == 63) wsum[wv] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wv; ++i) base += wsum[i];
    int pos = row_ptr[(size_t)h * nb + I] + base + incl - c;
    for (int J = a0; J < a1; ++J)
      if (rank[J] < kk || J == I) col_idx[pos++] = J;
    __syncthreads();   // wsum reused by the next head
  }
}

size_t select_ws_bytes(const LaunchArgs& a, const SeqTable& t) {   // row lengths + the order
  return 2 * align_up((size_t)a.H * t.blk[t.n] * sizeof(int32_t), 256);
}

hipError_t launch_select(const LaunchArgs& a, const SeqTable& t, const float* scores,
                         const int32_t* k_h, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* row_order, void* ws, hipStream_t stream) {
  const int rows = a.H * t.blk[t.n];        // CSR rows of every sequence, one after another
  const int nb = max_blocks(t);
  int32_t* counts = (int32_t*)ws;
  int32_t* tmp = (int32_t*)((char*)ws + align_up((size_t)rows * sizeof(int32_t), 256));
  hipLaunchKernelGGL(select_count_kernel, dim3((a.G * t.blk[t.n] + 3) / 4), dim3(256), 0, stream,
                     scores, k_h, counts, a.H, a.G, a.ratio, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int max_len = nb + 1;   // a row keeps at most I + 1 <= nb blocks
  hipLaunchKernelGGL(select_scan_kernel, dim3(1), dim3(kScanThreads),
                     row_order ? (size_t)(max_len + 1) * sizeof(int) : 0, stream, counts, row_ptr,
                     row_order, tmp, rows, max_len);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int Pmax = 1;
  while (Pmax < nb) Pmax <<= 1;
  const size_t smem = (size_t)Pmax * 8 + align_up((size_t)nb * 2, 16);
  hipLaunchKernelGGL(select_emit_kernel, dim3(a.G * t.blk[t.n]), dim3(kEmitThreads), smem, stream,
                     scores, k_h, row_ptr, col_idx, a.H, a.G, Pmax, a.ratio, t);
  return hipGetLastError();
}

}  // namespace pxa
