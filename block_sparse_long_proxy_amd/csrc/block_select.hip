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
//   select_chunk_sum / select_rowptr / select_schedule: exclusive scan of the
//     H*nb lengths -> row_ptr, and the XCD-aware, longest-first schedule of
//     the rows -> row_order (one workgroup per XCD).
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

// row_ptr and the attention schedule row_order.  Workgroup b of an attention
// launch goes to XCD b mod 8, and each XCD has its own L2, so the schedule is
// built per XCD:
//   * XCD x owns the rows whose midpoint in the cumulative work row_ptr falls
//     in the x-th eighth.  Rows are numbered h * nb + I and the heads of one
//     KV head are consecutive, so each XCD sees one or two KV heads and their
//     K/V tiles stay in its L2;
//   * position p of row_order is dealt to XCD p mod 8, so XCD x holds exactly
//     cap_x = ceil-or-floor(n / 8) positions; its own rows fill them longest
//     first, a surplus (its shortest rows) moves to XCDs with spare positions.
// Three launches: per-chunk sums of the lengths; the exclusive scan into
// row_ptr, which also records where each XCD's (contiguous) range of rows
// starts; one workgroup per XCD counting-sorts its rows by length (rows of
// equal length in no fixed order) and writes their positions.
constexpr int kXcds = 8;
constexpr int kScanWG = 256;                   // threads of the scan launches
constexpr int kRowsPerThread = 16;
constexpr int kChunkRows = kScanWG * kRowsPerThread;
constexpr int kSchedThreads = 1024;

__device__ __forceinline__ int xcd_of_row(int64_t start, int len, int64_t total) {
  // midpoint (start + len/2) scaled to [0, 8)
  const int64_t x = ((2 * start + len) * kXcds) / (2 * total);
  return (int)min<int64_t>(x, kXcds - 1);
}

// Sum over the workgroup (kScanWG threads); every thread gets the result.
__device__ __forceinline__ int block_sum(int v, int* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();                              // sh may still be read by a previous call
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kScanWG / 64; ++w) t += sh[w];
  return t;
}

// Exclusive prefix of v over the workgroup's threads (kScanWG of them).
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (l >= o) incl += y;
  }
  __syncthreads();
  if (l == 63) sh[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  return base + incl - v;
}

// Launch 1: part[c] = sum of the lengths of chunk c (kChunkRows rows).
__global__ __launch_bounds__(kScanWG) void select_chunk_sum_kernel(const int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ part, int n) {
  __shared__ int sh[kScanWG / 64];
  const int a = blockIdx.x * kChunkRows + threadIdx.x * kRowsPerThread;
  int v[kRowsPerThread];
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) v[k] = a + k < n ? counts[a + k] : 0;
  int s = 0;
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) s += v[k];
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// Launch 2: row_ptr (exclusive scan of the lengths, row_ptr[n] = total) and,
// with `bound`, bound[x] = the first row whose owner XCD is >= x (bound[8] = n).
__global__ __launch_bounds__(kScanWG) void select_rowptr_kernel(const int32_t* __restrict__ counts,
                                                                const int32_t* __restrict__ part,
                                                                int32_t* __restrict__ row_ptr,
                                                                int32_t* __restrict__ bound, int n,
                                                                int nchunks) {
  __shared__ int sh[kScanWG / 64];
  const int c = blockIdx.x;
  int off = 0, tot = 0;
  for (int i = threadIdx.x; i < nchunks; i += kScanWG) {
    const int p = part[i];
    tot += p;
    off += i < c ? p : 0;
  }
  off = block_sum(off, sh);
  tot = block_sum(tot, sh);
  const int a = c * kChunkRows + threadIdx.x * kRowsPerThread;
  int v[kRowsPerThread];
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) v[k] = a + k < n ? counts[a + k] : 0;
  int s = 0;
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) s += v[k];
  int run = off + block_exclusive_scan(s, sh);
  // owner XCD of the row before this thread's first row (-1 before row 0)
  int prev_owner = -1;
  if (bound && a > 0 && a < n) {
    const int len = counts[a - 1];
    prev_owner = xcd_of_row(run - len, len, tot);
  }
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int r = a + k;
    if (r >= n) break;
    row_ptr[r] = run;
    if (bound) {
      const int owner = xcd_of_row(run, v[k], tot);
      for (int x = prev_owner + 1; x <= owner; ++x) bound[x] = r;
      if (r == n - 1)
        for (int x = owner + 1; x <= kXcds; ++x) bound[x] = n;
      prev_owner = owner;
    }
    run += v[k];
    if (r == n - 1) row_ptr[n] = run;
  }
}

// Launch 3: one workgroup per XCD x.  Its rows [bound[x], bound[x+1]) get
// ranks by a counting sort on length, longest first; rank < cap_x takes
// position 8 rank + x, the surplus (its shortest rows) the spare positions of
// XCDs with fewer rows than positions, in XCD order.  hist: max_len + 1 ints
// of dynamic LDS.
__global__ __launch_bounds__(kSchedThreads) void select_schedule_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ bound,
    int32_t* __restrict__ row_order, int n, int max_len) {
  extern __shared__ int hist[];                 // [max_len + 1]
  __shared__ int lo[kXcds + 1];
  __shared__ int part[kSchedThreads / 64];
  const int x = blockIdx.x, t = threadIdx.x;
  if (t <= kXcds) lo[t] = bound[t];
  for (int c = t; c <= max_len; c += kSchedThreads) hist[c] = 0;
  __syncthreads();
  const int a = lo[x], b = lo[x + 1];
  for (int r = a + t; r < b; r += kSchedThreads) atomicAdd(&hist[min(counts[r], max_len)], 1);
  __syncthreads();
  {   // bucket starts, longest first: exclusive scan of hist from c = max_len down
    const int nbk = max_len + 1;
    const int per = (nbk + kSchedThreads - 1) / kSchedThreads;
    const int q0 = min(nbk, t * per), q1 = min(nbk, q0 + per);
    int sum = 0;
    for (int q = q0; q < q1; ++q) sum += hist[max_len - q];
    const int l = t & 63, w = t >> 6;
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    if (l == 63) part[w] = incl;
    __syncthreads();
    int acc = incl - sum;
    for (int i = 0; i < w; ++i) acc += part[i];
    for (int q = q0; q < q1; ++q) {
      const int hx = hist[max_len - q];
      hist[max_len - q] = acc;
      acc += hx;
    }
  }
  __syncthreads();
  // per-XCD counts, capacities and where the surplus goes (the same in every thread)
  int cnt[kXcds], cap[kXcds], deficit_start[kXcds + 1];
  int surplus_before = 0;
  deficit_start[0] = 0;
#pragma unroll
  for (int y = 0; y < kXcds; ++y) {
    cnt[y] = lo[y + 1] - lo[y];
    cap[y] = n / kXcds + (y < n % kXcds ? 1 : 0);
    deficit_start[y + 1] = deficit_start[y] + max(0, cap[y] - cnt[y]);
    if (y < x) surplus_before += max(0, cnt[y] - cap[y]);
  }
  for (int r = a + t; r < b; r += kSchedThreads) {
    const int rank = atomicAdd(&hist[min(counts[r], max_len)], 1);
    int pos;
    if (rank < cap[x]) {
      pos = kXcds * rank + x;
    } else {
      const int sj = surplus_before + rank - cap[x];
      int y = 0;
      while (y < kXcds - 1 && sj >= deficit_start[y + 1]) ++y;
      pos = kXcds * (cnt[y] + sj - deficit_start[y]) + y;
    }
    row_order[pos] = r;
  }
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

// row lengths, then the chunk sums and the XCD bounds (at most
// ceil(rows / kChunkRows) + 9 <= rows ints when rows > kChunkRows, and fewer
// than the part's 256-byte minimum otherwise)
size_t select_ws_bytes(const LaunchArgs& a, const SeqTable& t) {
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
  const int nchunks = (rows + kChunkRows - 1) / kChunkRows;
  hipLaunchKernelGGL(select_chunk_sum_kernel, dim3(nchunks), dim3(kScanWG), 0, stream, counts, tmp,
                     rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int32_t* bound = row_order ? tmp + nchunks : nullptr;     // kXcds + 1 entries
  hipLaunchKernelGGL(select_rowptr_kernel, dim3(nchunks), dim3(kScanWG), 0, stream, counts, tmp,
                     row_ptr, bound, rows, nchunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (row_order) {
    hipLaunchKernelGGL(select_schedule_kernel, dim3(kXcds), dim3(kSchedThreads),
                       (size_t)(max_len + 1) * sizeof(int), stream, counts, bound, row_order, rows,
                       max_len);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int Pmax = 1;
  while (Pmax < nb) Pmax <<= 1;
  const size_t smem = (size_t)Pmax * 8 + align_up((size_t)nb * 2, 16);
  hipLaunchKernelGGL(select_emit_kernel, dim3(a.G * t.blk[t.n]), dim3(kEmitThreads), smem, stream,
                     scores, k_h, row_ptr, col_idx, a.H, a.G, Pmax, a.ratio, t);
  return hipGetLastError();
}

}  // namespace pxa
