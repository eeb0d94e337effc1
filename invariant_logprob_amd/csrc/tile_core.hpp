// Shared core of the bf16 MFMA tile kernels (gfx950): the 256 x 256 tile
// geometry, the direct global -> LDS loader, the swizzled fragment reads and
// the K main loop.  Every tile kernel of the library forms its products
// through these pieces, so a tile's fp32 result depends only on its operand
// rows and on K -- never on the kernel, launch or batch that computes it.
//
// A tile multiplies kBP rows of operand P (the MFMA "M" side) by kBQ rows of
// operand Q (the MFMA "N" side); both operands are bf16 rows with K
// contiguous, and K is visited in ascending 64-wide stages, 16 per
// v_mfma_f32_32x32x16_bf16 instruction, accumulating in fp32.  Eight waves
// (two per SIMD) split the tile 2 (P) x 4 (Q); each wave owns 128 x 64 =
// 4 x 2 MFMA blocks.  Result layout of a 32 x 32 block: lane l holds Q row
// (l & 31) and P rows 8 (e >> 2) + 4 (l >> 5) + (e & 3), e = 0 .. 15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"

namespace rlk {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBP = 256;                // P rows per tile
constexpr int kBQ = 256;                // Q rows per tile
constexpr int kBK = kLinearKStage;      // K per pipeline stage
constexpr int kWaves = 8;               // 2 (P) x 4 (Q), two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWQ = kWaves / 2;         // waves along Q
constexpr int kQW = kBQ / kWQ;          // Q rows per wave (64)
constexpr int kPW = kBP / 2;            // P rows per wave (128)
constexpr int kJ = kQW / 32;            // 32-row Q blocks per wave (2)
constexpr int kI = kPW / 32;            // 32-row P blocks per wave (4)
constexpr int kRowChunks = kBK / 8;     // 16-byte chunks per tile row per stage
constexpr int kPVec = kBP * kRowChunks; // uint4 per stage, P side
constexpr int kQVec = kBQ * kRowChunks; // uint4 per stage, Q side
constexpr int kStageVec = kPVec + kQVec;
constexpr int kBlkPerWave = (kPVec / 64) / kWaves;  // 1 KB copies per wave per operand per stage
constexpr int kSub = kBK / 16;          // 16-deep MFMA steps per stage
static_assert(kPVec == kQVec, "loader assumes square tiles");
static_assert(kRowChunks == 8, "swizzle assumes 8 chunks per row");
static_assert(kBlkPerWave % 2 == 0, "a stage's copies are issued in two halves");
static_assert(2 * kStageVec * 16 <= 160 * 1024, "LDS budget of one CU");

// Word 3 of a raw buffer resource on gfx9-family parts (data format field)
constexpr int kBufferResourceWord3 = 0x00020000;
// A byte offset beyond any buffer range: such loads return zero.
constexpr int kOutOfRange = 0x7ffffff0;

// Raw buffer resource over [base, base + bytes), built from wave-uniform
// values so that it lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint16_t* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  void* q = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, n, kBufferResourceWord3);
}

// LDS chunk swizzle: chunk c of tile row r is stored at c ^ ((r >> 1) & 7) so
// that the 16-byte fragment reads of consecutive rows spread over all banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
// generic pointer into __shared__ memory -> LDS address space pointer
__device__ __forceinline__ lds_void_ptr to_lds(uint4* p) { return (lds_void_ptr)(p); }

// Per-lane loader state.  One wave instruction fills 1 KB of LDS = 8 tile
// rows of 128 bytes; lane l writes physical chunk (l & 7) of its row, which
// holds logical chunk (l & 7) ^ swizzle(row).  Each lane's byte offset is
// fixed for the whole K loop; a stage's K position goes into the scalar
// offset.
struct Loader {
  int voff_p[kBlkPerWave];
  int voff_q[kBlkPerWave];
  int kcol[kBlkPerWave];
};

__device__ __forceinline__ Loader make_loader(int wave, int lane, int64_t ldp, int64_t ldq) {
  Loader L;
#pragma unroll
  for (int q = 0; q < kBlkPerWave; ++q) {
    const int idx = (wave * kBlkPerWave + q) * 64 + lane;
    const int r = idx / kRowChunks;
    const int c = (idx % kRowChunks) ^ ((r >> 1) & 7);
    L.kcol[q] = 8 * c;
    L.voff_p[q] = (r * static_cast<int>(ldp) + 8 * c) * 2;
    L.voff_q[q] = (r * static_cast<int>(ldq) + 8 * c) * 2;
  }
  return L;
}

// Copies [Q0, Q1) of this wave for K stage kt into LDS stage buffer st.
// Rows past the operand's range (the resource's byte count) read as zero; in
// a ragged last stage, chunks at or past K are forced out of range (zero).
template <int Q0, int Q1>
__device__ __forceinline__ void issue(uint4* smem, const Loader& L, int wave,
                                      __amdgpu_buffer_rsrc_t pres, __amdgpu_buffer_rsrc_t qres,
                                      int kt, int st, int K) {
  const int k0 = kt * kBK;
  const bool full = (k0 + kBK) <= K;
  uint4* a = smem + st * kStageVec;
  uint4* b = a + kPVec;
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    const int blk = wave * kBlkPerWave + q;
    int vp = L.voff_p[q], vq = L.voff_q[q];
    if (!full && (k0 + L.kcol[q]) >= K) {
      vp = kOutOfRange;
      vq = kOutOfRange;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pres, to_lds(a + blk * 64), 16, vp, k0 * 2, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qres, to_lds(b + blk * 64), 16, vq, k0 * 2, 0, 0);
  }
}

// MFMA operands of one 16-deep step: lane supplies row (lane & 31) and
// k-chunk (lane >> 5) of each 32-row block.
__device__ __forceinline__ void frag(const uint4* a, int kk, int wp, int wq, int lane,
                                     bf16x8_t (&fa)[kI], bf16x8_t (&fb)[kJ]) {
  const uint4* b = a + kPVec;
  const int c = 2 * kk + (lane >> 5);
#pragma unroll
  for (int i = 0; i < kI; ++i) {
    const int r = wp * kPW + i * 32 + (lane & 31);
    fa[i] = __builtin_bit_cast(bf16x8_t, a[r * kRowChunks + swz(r, c)]);
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int r = wq * kQW + j * 32 + (lane & 31);
    fb[j] = __builtin_bit_cast(bf16x8_t, b[r * kRowChunks + swz(r, c)]);
  }
}

__device__ __forceinline__ void mma(f32x16_t (&acc)[kI][kJ], const bf16x8_t (&fa)[kI],
                                    const bf16x8_t (&fb)[kJ]) {
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16_t (&acc)[kI][kJ]) {
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// One stage's MFMA work with the copies of the stage after it issued in two
// halves during the first two steps (the caller's callbacks pf0 / pf1).
template <typename Pf0, typename Pf1>
__device__ __forceinline__ void stage(f32x16_t (&acc)[kI][kJ], const uint4* a, int wp, int wq,
                                      int lane, Pf0&& pf0, Pf1&& pf1) {
  bf16x8_t fa0[kI], fb0[kJ], fa1[kI], fb1[kJ];
  frag(a, 0, wp, wq, lane, fa0, fb0);
#pragma unroll
  for (int kk = 0; kk < kSub; kk += 2) {
    frag(a, kk + 1, wp, wq, lane, fa1, fb1);
    if (kk == 0) pf0();
    mma(acc, fa0, fb0);
    if (kk + 2 < kSub) frag(a, kk + 2, wp, wq, lane, fa0, fb0);
    if (kk == 0) pf1();
    mma(acc, fa1, fb1);
  }
}

// Whole-K main loop of one tile through two LDS buffers.  At the top of
// stage kt each wave waits for its own copies of stage kt, and the barrier
// makes every wave's copies visible (and frees the other buffer); stage
// kt + 1's copies are issued during the first two MFMA steps.  The wait and
// the barrier form one asm statement so that no LDS read can be scheduled
// between them.  Ends with a barrier: the LDS may be reused at once.
__device__ __forceinline__ void mainloop(uint4* smem, const Loader& L, int wave, int lane, int wp,
                                         int wq, __amdgpu_buffer_rsrc_t pres,
                                         __amdgpu_buffer_rsrc_t qres, int K,
                                         f32x16_t (&acc)[kI][kJ]) {
  const int n_kt = (K + kBK - 1) / kBK;
  zero(acc);
  issue<0, kBlkPerWave>(smem, L, wave, pres, qres, 0, 0, K);
  for (int kt = 0; kt < n_kt; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const bool pf = (kt + 1) < n_kt;
    const int nb = (kt + 1) & 1;
    stage(
        acc, smem + (kt & 1) * kStageVec, wp, wq, lane,
        [&] {
          if (pf) issue<0, kBlkPerWave / 2>(smem, L, wave, pres, qres, kt + 1, nb, K);
        },
        [&] {
          if (pf) issue<kBlkPerWave / 2, kBlkPerWave>(smem, L, wave, pres, qres, kt + 1, nb, K);
        });
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Operands in either layout.  A tile side (P or Q) reads its operand as
//   Lay::kRows  the side's tile rows are operand rows with K contiguous (the
//               layout above), or
//   Lay::kCols  the operand is stored K-major: operand row k holds the side's
//               tile rows as contiguous columns (W [V, H] contracted over V,
//               hidden [N, H] or D [N, C] contracted over N).
// A kCols stage sits in LDS as 64 K rows of 256 entries (512 B), 16-byte
// chunk c of row k stored at c ^ 4 (k & 3).  Its MFMA fragments come from
// transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane group, a
// lane that addresses row kb + s / 4, columns mb + 4 (s % 4) .. + 3 (s = the
// lane's index in its group) makes lane i of the group receive rows kb .. kb +
// 3 of column mb + i -- four consecutive K of one tile row, so two such reads
// give the eight K of a fragment.  The swizzle puts the four rows of a read
// in four different 64-byte bank ranges.

enum class Lay { kRows, kCols };

// One operand of a tile.  kRows: ptr = the tile's first row, extent = tile
// rows present (rows past it read as zero).  kCols: ptr = element (k = 0,
// column col0), the tile's first column; extent = K rows present.  A stage's
// resource ends where row min(extent, k0 + 64) starts, so nothing past the
// operand is read: bytes past it read as zero, and columns past the
// operand's width feed only output entries that are never stored.
struct Side {
  const uint16_t* ptr;
  int64_t ld;
  int extent;
  int col0;
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

__device__ __forceinline__ int swz_cols(int k, int c) { return c ^ (4 * (k & 3)); }

template <Lay LP, Lay LQ>
struct LoaderG {
  int voff_p[kBlkPerWave];
  int voff_q[kBlkPerWave];
  int kcol_p[kBlkPerWave];
  int kcol_q[kBlkPerWave];
};

template <Lay L>
__device__ __forceinline__ void lane_offset(int idx, int64_t ld, int& voff, int& kcol) {
  if constexpr (L == Lay::kRows) {
    const int r = idx / kRowChunks;
    const int c = (idx % kRowChunks) ^ ((r >> 1) & 7);
    kcol = 8 * c;
    voff = (r * static_cast<int>(ld) + 8 * c) * 2;
  } else {
    const int k = idx / 32;  // 32 chunks of 16 bytes per 256-entry row
    const int c = swz_cols(k, idx % 32);
    kcol = 0;
    voff = (k * static_cast<int>(ld) + 8 * c) * 2;
  }
}

template <Lay LP, Lay LQ>
__device__ __forceinline__ LoaderG<LP, LQ> make_loader_g(int wave, int lane, int64_t ldp,
                                                         int64_t ldq) {
  LoaderG<LP, LQ> L;
#pragma unroll
  for (int q = 0; q < kBlkPerWave; ++q) {
    const int idx = (wave * kBlkPerWave + q) * 64 + lane;
    lane_offset<LP>(idx, ldp, L.voff_p[q], L.kcol_p[q]);
    lane_offset<LQ>(idx, ldq, L.voff_q[q], L.kcol_q[q]);
  }
  return L;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// The four words of a raw buffer resource over [base, base + bytes) (stride
// 0), from wave-uniform values so that they live in scalar registers.
__device__ __forceinline__ i32x4_t uniform_desc(const uint16_t* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t d;
  d.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  d.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));
  d.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  d.w = kBufferResourceWord3;
  return d;
}

// Buffer resource and scalar offset of one side for the stage starting at k0.
template <Lay L>
__device__ __forceinline__ i32x4_t side_desc(const Side& s, int k0, int& soff) {
  if constexpr (L == Lay::kRows) {
    soff = k0 * 2;
    return uniform_desc(s.ptr, static_cast<int64_t>(s.extent) * s.ld * 2);
  } else {
    soff = 0;
    const int rows = min(max(s.extent - k0, 0), kBK);
    const int64_t elems = rows > 0 ? static_cast<int64_t>(rows) * s.ld - s.col0 : 0;
    return uniform_desc(s.ptr + static_cast<int64_t>(k0) * s.ld, elems * 2);
  }
}

// One wave's 16-byte-per-lane copy from a buffer into the LDS at dst (lane l
// writes dst + 16 l), written as the instruction itself.  The compiler,
// seeing a direct-to-LDS load through its builtin, makes every later
// transposing LDS read wait for it (vmcnt(0)) although the two touch
// different stage buffers; the caller's stage-top wait and barrier are what
// make the copied data visible.
__device__ __forceinline__ void copy16_to_lds(i32x4_t desc, uint4* dst, int voff, int soff) {
  const int m = __builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<uintptr_t>(to_lds(dst))));
  // M0 holds the LDS destination (an input bound to that register); one
  // wait state separates the M0 write from the copy that reads it
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(soff), "{m0}"(m)
      : "memory");
}

template <int Q0, int Q1, Lay LP, Lay LQ>
__device__ __forceinline__ void issue_g(uint4* smem, const LoaderG<LP, LQ>& L, int wave,
                                        const Side& P, const Side& Q, int kt, int st, int K) {
  const int k0 = kt * kBK;
  const bool full = (k0 + kBK) <= K;
  uint4* a = smem + st * kStageVec;
  uint4* b = a + kPVec;
  int sp, sq;
  const i32x4_t pres = side_desc<LP>(P, k0, sp);
  const i32x4_t qres = side_desc<LQ>(Q, k0, sq);
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    const int blk = wave * kBlkPerWave + q;
    int vp = L.voff_p[q], vq = L.voff_q[q];
    if constexpr (LP == Lay::kRows) {
      if (!full && (k0 + L.kcol_p[q]) >= K) vp = kOutOfRange;
    }
    if constexpr (LQ == Lay::kRows) {
      if (!full && (k0 + L.kcol_q[q]) >= K) vq = kOutOfRange;
    }
    copy16_to_lds(pres, a + blk * 64, vp, sp);
    copy16_to_lds(qres, b + blk * 64, vq, sq);
  }
}

// Fragment of 32-row block starting at tile row r0 for 16-deep step kk.
template <Lay L>
__device__ __forceinline__ bf16x8_t frag_side(const uint4* base, int kk, int r0, int lane) {
  if constexpr (L == Lay::kRows) {
    const int c = 2 * kk + (lane >> 5);
    const int r = r0 + (lane & 31);
    return __builtin_bit_cast(bf16x8_t, base[r * kRowChunks + swz(r, c)]);
  } else {
    const int g = lane >> 4;
    const int s = lane & 15;
    const int m = r0 + 16 * (g & 1) + 4 * (s & 3);
    const char* bytes = reinterpret_cast<const char*>(base);
    s16x4_t h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int k = 16 * kk + 8 * (g >> 1) + 4 * t + (s >> 2);
      const char* p = bytes + k * 512 + 16 * swz_cols(k, m >> 3) + 2 * (m & 7);
      h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    }
    const uint4 u = make_uint4(__builtin_bit_cast(uint2, h[0]).x, __builtin_bit_cast(uint2, h[0]).y,
                               __builtin_bit_cast(uint2, h[1]).x, __builtin_bit_cast(uint2, h[1]).y);
    return __builtin_bit_cast(bf16x8_t, u);
  }
}

template <Lay LP, Lay LQ>
__device__ __forceinline__ void frag_g(const uint4* a, int kk, int wp, int wq, int lane,
                                       bf16x8_t (&fa)[kI], bf16x8_t (&fb)[kJ]) {
  const uint4* b = a + kPVec;
#pragma unroll
  for (int i = 0; i < kI; ++i) fa[i] = frag_side<LP>(a, kk, wp * kPW + i * 32, lane);
#pragma unroll
  for (int j = 0; j < kJ; ++j) fb[j] = frag_side<LQ>(b, kk, wq * kQW + j * 32, lane);
}

// The main loop of `mainloop` for operands in any layout: same stage order,
// same double buffering, same MFMA sequence.  With zero_acc false the
// products are added to the accumulators' current values (a second pass over
// the same K, continuing the same fixed order).
template <Lay LP, Lay LQ>
__device__ __forceinline__ void mainloop_g(uint4* smem, const LoaderG<LP, LQ>& L, int wave,
                                           int lane, int wp, int wq, const Side& P, const Side& Q,
                                           int K, f32x16_t (&acc)[kI][kJ], bool zero_acc = true) {
  const int n_kt = (K + kBK - 1) / kBK;
  if (zero_acc) zero(acc);
  if (n_kt <= 0) return;
  issue_g<0, kBlkPerWave>(smem, L, wave, P, Q, 0, 0, K);
  for (int kt = 0; kt < n_kt; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const bool pf = (kt + 1) < n_kt;
    const int nb = (kt + 1) & 1;
    const uint4* a = smem + (kt & 1) * kStageVec;
    bf16x8_t fa0[kI], fb0[kJ], fa1[kI], fb1[kJ];
    frag_g<LP, LQ>(a, 0, wp, wq, lane, fa0, fb0);
#pragma unroll
    for (int kk = 0; kk < kSub; kk += 2) {
      frag_g<LP, LQ>(a, kk + 1, wp, wq, lane, fa1, fb1);
      if (kk == 0 && pf) issue_g<0, kBlkPerWave / 2>(smem, L, wave, P, Q, kt + 1, nb, K);
      mma(acc, fa0, fb0);
      if (kk + 2 < kSub) frag_g<LP, LQ>(a, kk + 2, wp, wq, lane, fa0, fb0);
      if (kk == 0 && pf) issue_g<kBlkPerWave / 2, kBlkPerWave>(smem, L, wave, P, Q, kt + 1, nb, K);
      mma(acc, fa1, fb1);
    }
  }
  __syncthreads();
}

// Element idx = 16 i + e of column block j of the accumulators, for a
// per-lane idx in [0, 64): a six-level select tree on the bits of idx, so
// that each level shares one lane mask.  Each bit passes through an empty
// asm statement: seen as the bits of one index, the tree can be folded back
// into an indexed read, which puts the accumulators in scratch memory.
template <int NJ>
__device__ __forceinline__ float select_acc(const f32x16_t (&acc)[kI][NJ], int j, int idx) {
  static_assert(kI * 16 == 64, "select tree is sized for 64 elements per column block");
  int bit[6];
#pragma unroll
  for (int lvl = 0; lvl < 6; ++lvl) {
    bit[lvl] = (idx >> lvl) & 1;
    asm volatile("" : "+v"(bit[lvl]));
  }
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int a = 2 * k, b = 2 * k + 1;
    v[k] = bit[0] ? acc[b >> 4][j][b & 15] : acc[a >> 4][j][a & 15];
  }
#pragma unroll
  for (int lvl = 1, n = 16; lvl < 6; ++lvl, n >>= 1)
#pragma unroll
    for (int k = 0; k < n; ++k) v[k] = bit[lvl] ? v[2 * k + 1] : v[2 * k];
  return v[0];
}

// Launch-order regrouping: workgroups are dispatched round-robin over the 8
// XCDs, so ids are first regrouped into contiguous per-XCD ranges; within a
// range, tiles go by groups of `group` major tiles x all minor tiles, so the
// workgroups sharing an XCD (and its L2) work on few operand slabs at a
// time.  A bijection on [0, n_major * n_minor); it only decides *when* a
// tile runs, never how it is computed.
__device__ __forceinline__ void grouped_coords(int w, int n_major, int n_minor, int group,
                                               int& major, int& minor) {
  const int total = n_major * n_minor;
  const int t8 = (total / 8) * 8;
  int L = w;
  if (w < t8) L = (w & 7) * (t8 / 8) + (w >> 3);
  const int span = group * n_minor;
  const int g = L / span;
  const int rem = L - g * span;
  const int gsize = min(group, n_major - g * group);
  minor = rem / gsize;
  major = g * group + (rem - minor * gsize);
}

}  // namespace tile
}  // namespace rlk
