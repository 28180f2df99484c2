// pxa_device.hpp -- device building blocks shared by the gfx950 kernels.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64,
// lane l, hi = l / 32):
//   A (32 x 16, M x K): lane holds A[l % 32][8*hi .. 8*hi+7]
//   B (16 x 32, K x N): lane holds B[8*hi .. 8*hi+7][l % 32]
//   C (32 x 32)       : register r holds C[8*(r/4) + 4*hi + r%4][l % 32]
//
// Attention tiles are computed transposed: S^T = K . Q^T, so a lane owns one
// query column (n = l % 32) and 16 key rows per 32-key sub-tile.  Row-wise
// softmax statistics are then mostly in-lane, and the probabilities already
// sit in the B-operand layout of O^T += V^T . P^T (the key index is the
// contraction index, in the permuted order the C layout gives).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pxa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 128;     // key/query block edge (tokens)
constexpr int kWaves = 4;       // waves per workgroup in the tile kernels
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row-major [128][D] bf16 tile in LDS with a 16-byte-chunk XOR swizzle:
// chunk c of row r lives at chunk (c ^ (r & (D/8 - 1))).  A wave reading one
// chunk column from 32 consecutive rows touches every bank group once.
template <int D>
__device__ __forceinline__ int ktile_off(int row, int chunk) {
  constexpr int C = D / 8;
  return row * D + ((chunk ^ (row & (C - 1))) << 3);
}

// A operand (keys x d) of sub-tile `t` (32 keys) and k-step `s` (16 dims);
// T is the 16-bit element type (bf16 inputs or fp16 proxies).
template <int D, typename T = __bf16>
__device__ __forceinline__ T __attribute__((ext_vector_type(8))) ktile_frag(const T* lds, int t, int s) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  const int l = threadIdx.x & 63;
  const int row = t * 32 + (l & 31);
  const int chunk = 2 * s + (l >> 5);
  return *reinterpret_cast<const v8*>(lds + ktile_off<D>(row, chunk));
}

// B operand (d x queries) for k-step s, read straight from global memory:
// query row `qrow` (pointer to its first element), dims 16 s + 8 hi .. +7.
template <int D, typename T = __bf16>
__device__ __forceinline__ void load_qfrag(const T* __restrict__ qrow,
                                           T __attribute__((ext_vector_type(8))) (&qf)[D / 16]) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  const int hi = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = *reinterpret_cast<const v8*>(qrow + 16 * s + 8 * hi);
}

// S^T (128 keys x 32 queries of this wave) = K_tile . Q^T, four 32x32 tiles.
template <int D>
__device__ __forceinline__ void tile_scores(const __bf16* ks, const bf16x8 (&qf)[D / 16], f32x16 (&acc)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = zero16();
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mfma32(ktile_frag<D>(ks, t, s), qf[s], acc[t]);
  }
}

// Key index (0..127 inside the block) held by register r of sub-tile t.
__device__ __forceinline__ int acc_key(int t, int r) {
  const int hi = (threadIdx.x & 63) >> 5;
  return t * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
}

// ---------------------------------------------------------------------------
// Wave-level reductions (wave64).
// Max over the 64 lanes of a wave without LDS traffic: DPP moves reduce each
// row of 16 lanes, two row broadcasts fold the rows into lane 63, whose value
// is returned (wave-uniform).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max_uniform(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x, x));         // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_move<0x4E>(x, x));         // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_move<0x141>(x, x));        // row_half_mirror
  x = fmaxf(x, dpp_move<0x140>(x, x));        // row_mirror: every lane holds its row's max
  x = fmaxf(x, dpp_move<0x142, 0xA>(x, x));   // row_bcast:15 into rows 1 and 3
  x = fmaxf(x, dpp_move<0x143, 0xC>(x, x));   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sequence of a fused launch that holds item x: the s with pre[s] <= x <
// pre[s+1] (pre: one of the SeqTable prefix arrays, x < pre[n]).  Binary
// search on wave-uniform values, so it runs on scalar loads of the kernel
// arguments.
__device__ __forceinline__ int seq_find(const int32_t* pre, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Order-preserving map of a finite float to uint32 (larger float -> larger
// code); -0 is folded onto +0 first so that equal scores compare equal.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  f = f + 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sort key of block J with score s: ascending key order == score descending,
// then block index ascending.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t J) {
  return ((uint64_t)(~float_order_key(s)) << 32) | (uint64_t)J;
}

}  // namespace pxa

namespace pxa {

// ---------------------------------------------------------------------------
// Direct global -> LDS tile copies (global_load_lds_dwordx4: lane l of a wave
// writes its 16 bytes at LDS base + 16 l, so one instruction fills 1 KB, i.e.
// 1024 / (2 D) consecutive rows).  The source address of each lane is chosen
// so that the LDS image is the XOR-swizzled layout the readers expect; no
// registers and no VALU work are spent on staging.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short lds_s16;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Swizzle of 16-byte chunks for the K tile (MFMA A operand read with 16-byte
// loads, 32 consecutive rows per wave): chunk ^ (row mod chunks-per-row).
template <int D>
__device__ __forceinline__ int kswz(int row) { return row & (D / 8 - 1); }
// Swizzle for the V tile read with ds_read_b64_tr_b16 (16 lanes read 4
// consecutive rows x 32 bytes): rows 4k..4k+3 land on disjoint bank groups.
template <int D>
__device__ __forceinline__ int vswz(int row) { return (row & 3) * (D / 32); }

// A wave-uniform pointer moved into scalar registers (64-bit products of
// uniform values are formed in vector registers and would otherwise stay there).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One global_load_lds_dwordx4 in scalar-base mode: this lane's 16 bytes at
// gbase + voff go to LDS byte address lds_wave_base + 16 * lane.  Issued
// through asm so the compiler does not drain every pending copy before
// unrelated LDS reads (it cannot tell the destination tiles apart).  No
// register is written.  Ordering is explicit: every LDS access to a copy's
// destination tile is separated from the copy by a workgroup barrier (reads
// of the old contents before it; reads of the new contents after
// wait_vmem*() and the next barrier), and volatile asm keeps its place
// relative to those waits and barriers.  There is deliberately no "memory"
// clobber: it would forbid scalar loads of read-only arguments.
__device__ __forceinline__ void lds_dma16(const void* gbase_in, uint32_t voff, uint32_t lds_in) {
  // both bases are wave-uniform; readfirstlane puts them in SGPRs
  const void* gbase = uniform_ptr(gbase_in);
  const uint32_t lds_wave_base = __builtin_amdgcn_readfirstlane(lds_in);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_wave_base), "v"(voff), "s"(gbase)
      : "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Copy one [128][D] bf16 tile (rows D elements apart at g, wave-uniform) into
// the swizzled LDS image at lds, using NW waves.  Instruction it of wave w
// fills rows (it * NW + w) * ROWS .. +ROWS-1; the swizzle term depends on the
// row only modulo NW * ROWS (a multiple of 16), which is the same for every
// instruction of a wave, so one per-lane byte offset serves all of them and
// only the scalar base moves.
template <int D, bool IS_V, int NW = kWaves, typename T>
__device__ __forceinline__ void tile_load_lds(const T* __restrict__ g, T* lds) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  constexpr int C = D / 8;                    // 16-byte chunks per row
  constexpr int ROWS = 64 / C;                // rows per wave instruction
  constexpr int INSTS = kBlock / ROWS / NW;
  static_assert((NW * ROWS) % 16 == 0, "swizzle must repeat every instruction");
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) % NW;   // scalar
  const int l = threadIdx.x & 63;
  g = uniform_ptr(g);
  const int row0 = w * ROWS + l / C;          // row of instruction 0
  const int logical = (l % C) ^ (IS_V ? vswz<D>(row0) : kswz<D>(row0));
  const uint32_t voff = (uint32_t)((l / C) * D + logical * 8) * 2u;   // bytes, same for all it
  const uint32_t lbase = lds_addr(lds) + (uint32_t)(w * ROWS * D * 2);
#pragma unroll
  for (int it = 0; it < INSTS; ++it) {
    const int blk_row = (it * NW + w) * ROWS;
    lds_dma16(g + (size_t)blk_row * D, voff, lbase + (uint32_t)(it * NW * ROWS * D * 2));
  }
}

// The same copy for a partial tile (the last block of a sequence whose length
// 128 does not divide): only `rows` (1..127) rows exist at g; every LDS row
// past them receives a copy of row rows-1, so no address beyond the tile's
// last token is formed.  The source row now varies per instruction, so the
// per-lane offset is recomputed each time from the unchanged scalar base.
template <int D, bool IS_V, int NW = kWaves, typename T>
__device__ __forceinline__ void tile_load_lds_rows(const T* __restrict__ g, T* lds, int rows) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  constexpr int C = D / 8;
  constexpr int ROWS = 64 / C;
  constexpr int INSTS = kBlock / ROWS / NW;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) % NW;
  const int l = threadIdx.x & 63;
  g = uniform_ptr(g);
  const int row0 = w * ROWS + l / C;
  const int logical = (l % C) ^ (IS_V ? vswz<D>(row0) : kswz<D>(row0));
  const uint32_t lbase = lds_addr(lds) + (uint32_t)(w * ROWS * D * 2);
#pragma unroll
  for (int it = 0; it < INSTS; ++it) {
    const int src = min((it * NW + w) * ROWS + l / C, rows - 1);
    const uint32_t voff = (uint32_t)(src * D + logical * 8) * 2u;
    lds_dma16(g, voff, lbase + (uint32_t)(it * NW * ROWS * D * 2));
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Element offset of (row, col) in a swizzled V tile.
template <int D>
__device__ __forceinline__ int vtile_off(int row, int col) {
  return row * D + (((col >> 3) ^ vswz<D>(row)) << 3) + (col & 7);
}

// A operand of O^T += V^T . P^T from a row-major (keys x dims) V tile, read
// with the transposing LDS load: lane (group g16 = (l/16)%2, i = l%16) gets
// dim 32 m + 16 g16 + i and keys kb..kb+3 from one read, kb+8..kb+11 from the
// second, kb = 32 t + 16 s2 + 4 hi -- the keys the C layout of S^T sub-tile t
// gives this lane in registers 8 s2 .. 8 s2 + 7.
template <int D>
__device__ __forceinline__ bf16x8 vfrag_tr(const __bf16* vs, int m, int t, int s2) {
  const int l = threadIdx.x & 63;
  const int i = l & 15, g16 = (l >> 4) & 1, hi = l >> 5;
  const int col = 32 * m + 16 * g16 + 4 * (i & 3);
  const int row = 32 * t + 16 * s2 + 4 * hi + (i >> 2);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((lds_s16*)vs + vtile_off<D>(row, col)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((lds_s16*)vs + vtile_off<D>(row + 8, col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace pxa
