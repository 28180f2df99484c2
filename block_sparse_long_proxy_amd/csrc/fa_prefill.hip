// fa_prefill.hip -- block-sparse (and dense) causal prefill attention.
//
// ProxyAttn blog post (ir.hit.edu.cn), section 4, final step: the block
// sparse mask goes to FlashAttention; section 2: a kept block is a whole
// 128x128 tile so the tiled kernel can skip the rest.  O = softmax(scale QK^T)V
// restricted to kept blocks and j <= i, online softmax in fp32.
//
// One workgroup = one (head h, query block I); 4 waves x 32 queries.  For
// every kept key block J (diagonal first, then descending J) the K and V
// tiles are staged through LDS and the wave computes
//   S^T = K Q^T (32 MFMA 32x32x16), online softmax in registers,
//   O^T += V^T P^T (32 MFMA).
// K and V tiles are copied global -> LDS directly (no staging registers); the
// copy of the next tile is issued before the MFMA phase it hides behind (V
// during S + softmax, the next K during PV).  V stays row-major in LDS and is
// read transposed with ds_read_b64_tr_b16.  A partial last block (128 does
// not divide N) is read with its missing rows repeated from token N-1; the
// rows of a fused batch are numbered sequence by sequence.
#include <cmath>

#include "pxa_device.hpp"
#include "pxa_launch.hpp"

namespace pxa {

// Row max of a tile (this lane's 64 logits, then the lane holding the same query).
__device__ __forceinline__ float tile_row_max(const f32x16 (&s)[4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
  return fmaxf(mx, __shfl_xor(mx, 32, 64));
}

// Online-softmax update for one 128-key tile whose logits are in s[4]
// (S^T layout: this lane's query, 64 of the tile's keys) with tile max mx.
// Masked entries are -inf.  Returns the bf16 probabilities in the B-operand
// layout of the PV MFMA and rescales the running output when the running max
// moved.
template <int D>
__device__ __forceinline__ void softmax_update(f32x16 (&s)[4], float mx, bf16x8 (&pb)[4][2],
                                               f32x16 (&oacc)[D / 32], float& m_run,
                                               float& l_run, float scale_log2) {
  const float m_new = fmaxf(m_run, mx);
  // m_new is finite once any unmasked key has been seen (always true after
  // the diagonal block, which comes first when present).
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  // v_exp_f32 directly: probabilities below 2^-126 flush to zero.
  const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
  m_run = m_new;
  const float mb = m_use * scale_log2;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pb[t][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[t][r], scale_log2, -mb));
  // Row sum of the bf16 probabilities the PV product uses (two per dot2), so
  // the normaliser matches the numerator's weights exactly.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][s2][e], pb[t][s2][e + 1]}, ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[t][s2][e + 2], pb[t][s2][e + 3]}, ones, ls1, false);
      }
  l_run = fmaf(l_run, alpha, ls0 + ls1);
  if (__any(alpha != 1.0f)) {      // wave-uniform: skip when no max moved
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
  }
}

// Wave priorities (s_setprio) of the three phases of a step.  The two waves
// sharing a SIMD (one from each of the CU's two workgroups) run out of phase;
// when both can issue, the one in its softmax (the dependent VALU chain
// between the products) goes first, then one in its PV products, and the QK^T
// products of the other wave fill in behind.  Each switch also fences the
// compiler's schedule, so the exponentials are computed before the PV
// products rather than spread among them.
constexpr int kPrioScores = 0;
constexpr int kPrioSoftmax = 2;
constexpr int kPrioPV = 1;

// One pipeline step on key block J (tiles already in LDS / landing): S, the
// softmax, then O += V P, issuing the copies of block Jn (knext / vnext NULL:
// none; next_rows < 128: Jn is a partial last block).
// SKIP: the running-max skip of the BLASST pages -- when every query of the
// wave has its tile max below m_run + skip_delta (raw logit units), the wave
// drops the tile's softmax and PV product.  It is a template parameter so the
// kernels launched without a threshold carry none of its code.
template <int D, bool DIAG, bool SKIP>
__device__ __forceinline__ void fa_step(const __bf16* ks_lds, const __bf16* vs_lds, __bf16* ks,
                                        __bf16* vs, const bf16x8 (&qf)[D / 16],
                                        f32x16 (&oacc)[D / 32], float& m_run, float& l_run,
                                        float scale_log2, int qloc, const __bf16* knext,
                                        const __bf16* vnext, int next_rows, float skip_delta) {
  f32x16 s[4];
  // S^T = K Q^T with the four K fragments of k-step ss+1 read while the four
  // products of step ss issue (scheduling barriers keep that order).
  __builtin_amdgcn_s_setprio(kPrioScores);
  {
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = zero16();
    bf16x8 a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = ktile_frag<D>(ks_lds, t, 0);
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss) {
      bf16x8 an[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) an[t] = (ss + 1 < D / 16) ? ktile_frag<D>(ks_lds, t, ss + 1) : a[t];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = mfma32(a[t], qf[ss], s[t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = an[t];
    }
  }
  if (DIAG) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_key(t, r) > qloc) s[t][r] = -INFINITY;
  }
  __builtin_amdgcn_s_setprio(kPrioSoftmax);
  bf16x8 pb[4][2];
  const float mx = tile_row_max(s);
  // m_run is -inf only before the first tile, where the comparison is false
  const bool skip = SKIP && !DIAG && __all(mx < m_run + skip_delta);
  if (!skip) softmax_update<D>(s, mx, pb, oacc, m_run, l_run, scale_log2);

  wait_vmem();                   // this thread's part of V(J) has landed
  __syncthreads();               // V(J) visible; every wave is done with the K tile
  if (knext) {
    if (next_rows < kBlock) tile_load_lds_rows<D, false>(knext, ks, next_rows);
    else tile_load_lds<D, false>(knext, ks);
  }

  __builtin_amdgcn_s_setprio(kPrioPV);
  if (!skip) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int m = 0; m < D / 32; ++m)
          oacc[m] = mfma32(vfrag_tr<D>(vs_lds, m, t, s2), pb[t][s2], oacc[m]);
  }

  // Same priority again: the switch keeps every PV product ahead of the copy
  // wait and the barrier (left alone, the compiler sinks the last products
  // past them, which measured slower).
  __builtin_amdgcn_s_setprio(kPrioPV);
  wait_vmem();                   // this thread's part of K(Jn) has landed
  __syncthreads();               // K(Jn) visible; every wave is done with the V tile
  if (vnext) {
    if (next_rows < kBlock) tile_load_lds_rows<D, true>(vnext, vs, next_rows);
    else tile_load_lds<D, true>(vnext, vs);
  }
}

template <int D, bool DENSE, bool SKIP>
__global__ __launch_bounds__(kThreads, 2) void fa_prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ row_order, __bf16* __restrict__ o, int H, int Hkv,
    float scale_log2, float skip_delta, const SeqTable t) {
  __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * D];   // K tile, kswz layout
  __shared__ __attribute__((aligned(16))) __bf16 vs[kBlock * D];   // V tile, vswz layout

  // Rows of a fused batch are numbered sequence by sequence (H * nb_s rows
  // each, h * nb_s + I within the sequence).
  int sid, h, I, nb;
  if (!DENSE && row_order) {
    const int r = row_order[blockIdx.x];
    if (r < 0 || r >= H * t.blk[t.n]) return;
    sid = t.n == 1 ? 0 : seq_find(t.blk, t.n, r / H);
    nb = t.blk[sid + 1] - t.blk[sid];
    const int rr = r - H * t.blk[sid];
    h = rr / nb;
    I = rr % nb;
  } else {
    sid = t.n == 1 ? 0 : seq_find(t.blk, t.n, (int)blockIdx.x / H);
    nb = t.blk[sid + 1] - t.blk[sid];
    const int bl = (int)blockIdx.x - H * t.blk[sid];
    // Query blocks from last (longest causal row) to first.  Workgroups are
    // dealt round-robin to the 8 XCDs (XCD = blockIdx mod 8).  Dense: XCD x
    // gets the consecutive heads [x H/8, (x+1) H/8), i.e. whole KV-head groups
    // when H/8 is a multiple of H/Hkv, so heads reading the same K/V tiles at
    // the same time share that XCD's L2.  Sparse without a schedule: heads
    // have unequal work, so the head index is rotated by the query block and
    // every head visits every XCD.
    const int step = bl / H;
    I = nb - 1 - step;
    const int j = bl % H;
    if (DENSE)
      h = (H % 8 == 0) ? (j % 8) * (H / 8) + j / 8 : j;
    else
      h = (j + step) % H;
  }
  // wave-uniform indices in scalar registers, so tile addresses stay scalar
  h = __builtin_amdgcn_readfirstlane(h);
  I = __builtin_amdgcn_readfirstlane(I);
  const int kvh = __builtin_amdgcn_readfirstlane(h / (H / Hkv));
  const int N = t.tok[sid + 1] - t.tok[sid];
  const size_t tok0 = (size_t)t.tok[sid];
  q += tok0 * H * D;
  o += tok0 * H * D;
  k += tok0 * Hkv * D;
  v += tok0 * Hkv * D;
  const int row = H * t.blk[sid] + h * nb + I;   // CSR row
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int qloc = 32 * w + (l & 31);          // query index inside block I

  const __bf16* kbase = k + (size_t)kvh * N * D;
  const __bf16* vbase = v + (size_t)kvh * N * D;
  constexpr size_t kTile = (size_t)kBlock * D;

  // Queries past the end of a partial last block read token N-1 (their
  // outputs are never stored); that block's missing keys read token N-1 too
  // and are masked by causality for every query that exists.
  const int qtok = I * kBlock + qloc;
  bf16x8 qf[D / 16];
  load_qfrag<D>(q + ((size_t)h * N + (size_t)min(qtok, N - 1)) * D, qf);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) oacc[m] = zero16();
  float m_run = -INFINITY;   // running max of raw logits (this lane's query)
  float l_run = 0.f;         // this lane's partial row sum (its 64 keys / block)

  int beg, end;
  if (DENSE) {
    beg = 0;
    end = I + 1;
  } else {
    beg = row_ptr[row];
    end = row_ptr[row + 1];
  }
  // Next valid block at or below list position `it` (walking towards beg),
  // or -1.  The list is visited from its end: the diagonal block, the largest
  // valid index, comes first, so the running max is set early and only that
  // first step needs the causal mask.
  // (Indices are made explicitly wave-uniform so the entries come through the
  // scalar cache and never wait on the vector-memory counter, which also
  // counts the tile copies in flight.)
  auto next_block = [&](int& it) -> int {
    for (; it >= beg; --it) {
      const int J = DENSE ? it : __builtin_amdgcn_readfirstlane(col_idx[__builtin_amdgcn_readfirstlane(it)]);
      if (J >= 0 && J <= I) return J;
    }
    return -1;
  };

  // Tokens of key block J (fewer than 128 only in a partial last block, which
  // with ascending columns can only be this first tile; checked everywhere so
  // that no column list makes a copy read past the end of K or V).
  auto rows_of = [&](int J) { return min(kBlock, N - J * kBlock); };
  int it = end - 1;
  int J = next_block(it);
  if (J >= 0) {
    const int rows = rows_of(J);
    if (rows < kBlock) {
      tile_load_lds_rows<D, false>(kbase + (size_t)J * kTile, ks, rows);
      tile_load_lds_rows<D, true>(vbase + (size_t)J * kTile, vs, rows);
    } else {
      tile_load_lds<D, false>(kbase + (size_t)J * kTile, ks);
      tile_load_lds<D, true>(vbase + (size_t)J * kTile, vs);
    }
  }
  wait_vmem();
  __syncthreads();

  if (J == I) {
    --it;
    const int Jn = next_block(it);
    fa_step<D, true, SKIP>(ks, vs, ks, vs, qf, oacc, m_run, l_run, scale_log2, qloc,
                     Jn >= 0 ? kbase + (size_t)Jn * kTile : nullptr,
                     Jn >= 0 ? vbase + (size_t)Jn * kTile : nullptr,
                     Jn >= 0 ? rows_of(Jn) : kBlock, skip_delta);
    J = Jn;
  }
  while (J >= 0) {
    --it;
    const int Jn = next_block(it);
    fa_step<D, false, SKIP>(ks, vs, ks, vs, qf, oacc, m_run, l_run, scale_log2, qloc,
                      Jn >= 0 ? kbase + (size_t)Jn * kTile : nullptr,
                      Jn >= 0 ? vbase + (size_t)Jn * kTile : nullptr,
                      Jn >= 0 ? rows_of(Jn) : kBlock, skip_delta);
    J = Jn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qtok >= N) return;          // no barrier follows
  __bf16* orow = o + ((size_t)h * N + (size_t)qtok) * D;
  const int hi = l >> 5;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[m][4 * g4 + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * m + 8 * g4 + 4 * hi) = ov;
    }
  }
}

template <int D>
static hipError_t launch_fa(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                            const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                            const int32_t* row_order, void* o, bool dense, hipStream_t stream) {
  const dim3 grid(a.H * t.blk[t.n]), block(kThreads);
  const float sl2 = a.scale * kLog2e;
  // skip when scale * (tile max - running max) < ln(threshold)
  const bool skip = a.skip_threshold > 0.f;
  const float skip_delta = skip ? std::log(a.skip_threshold) / a.scale : -INFINITY;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, row_ptr, col_idx, row_order, (__bf16*)o, a.H, a.Hkv,
                       sl2, skip_delta, t);
  };
  if (dense) {
    if (skip) go(fa_prefill_kernel<D, true, true>);
    else go(fa_prefill_kernel<D, true, false>);
  } else {
    if (skip) go(fa_prefill_kernel<D, false, true>);
    else go(fa_prefill_kernel<D, false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_fa_prefill(const LaunchArgs& a, const SeqTable& t, const void* q, const void* k,
                             const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* row_order, void* o, bool dense, hipStream_t stream) {
  return a.D == 64 ? launch_fa<64>(a, t, q, k, v, row_ptr, col_idx, row_order, o, dense, stream)
                   : launch_fa<128>(a, t, q, k, v, row_ptr, col_idx, row_order, o, dense, stream);
}

}  // namespace pxa
