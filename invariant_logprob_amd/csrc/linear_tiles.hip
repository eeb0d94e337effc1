// Fused lm_head projection + selected logprob ("linear_logp") and its
// backward with respect to the logits, on bf16 MFMA (gfx950).
//
// The projection z = h . W^T is a dense contraction, so it runs on the
// matrix cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation, K = H visited in
// ascending 64-wide stages, 16 elements per instruction -- the same
// instruction sequence for every tile, every N and every row position.
// Operand roles: W rows (vocabulary) are the MFMA "M" side and hidden rows
// (tokens) the "N" side, so each lane of the result holds 16 vocabulary
// entries of one token and a token's log-sum-exp is mostly lane-local.
//
// Tile = 256 vocabulary entries x 256 tokens, 8 waves (two per SIMD, so one
// wave's MFMAs cover the other's LDS and copy work) as 2 (vocab) x 4
// (tokens), each wave 128 x 64 = 4 x 2 MFMA blocks.  A 256-wide vocabulary
// tile is also the reduction chunk: per token, the tile's 256 logits are
// reduced in a fixed order (lane-local ascending, then the two lane halves,
// then the two vocabulary waves) to one (M, s) partial, written to the
// workspace.  A second kernel merges a row's partials in a fixed order.
// Rows beyond N in the last token block are zero-filled and never written.
// The logits stay fp32 and are never rounded to bf16.
//
// The pages fix the contract these kernels keep: bitwise batch invariance
// (page "[RFC] Batch-Invariant RL Kernel Suite for Train-Inference
// Consistency", maintainer reply, relation I); fixed, shape-independent
// reduction order and no atomics (page "[WS1 Test] #154 dtype pin + ...",
// section "Workstream 3 - #153", scope item 2); bf16 inputs with fp32
// accumulation (same page, "Workstream 1 - #154" scope table).  The tile
// schedule, the MFMA instruction and the K order never depend on N (a batch
// of at most 128 rows runs the same per-row sequence in a smaller launch, in
// the forward and in the backward).
//
// The backward kernel runs the same per-tile main loop (same copies, same
// MFMA sequence), so its z is bit-identical to the forward's, and replaces
// the epilogue by d = g (onehot - 2^(z log2 e - lse log2 e)).  A caller that
// can hold N x V fp32 may instead have the forward keep its logits (the
// kStoreLogits instantiation) and form the same gradient from them with an
// elementwise pass (logits_rows.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"
#include "tile_core.hpp"

namespace rlk {

namespace {

using namespace tile;

constexpr int kBV = kLinearVocabTile;   // vocabulary entries per tile (= chunk): the P side
constexpr int kBT = kLinearTokenTile;   // tokens per tile: the Q side
constexpr int kStageStride = 132;       // floats per staged output row (128 + 4 pad)
constexpr int kStagingVec = kWaves * 32 * kStageStride / 4;
constexpr int kSmemVec = (2 * kStageVec > kStagingVec) ? 2 * kStageVec : kStagingVec;
static_assert(kBV == kBP && kBT == kBQ, "vocabulary rows are the P side, tokens the Q side");
static_assert(kSmemVec * 16 <= 160 * 1024, "LDS budget of one CU");

struct TileArgs {
  const uint16_t* hidden;
  int64_t ldh;
  const uint16_t* weight;
  int64_t ldw;
  const int64_t* targets;
  const uint8_t* mask;
  int64_t N;
  int V;
  int H;
  int n_vtiles;
  int n_tblocks;
  // forward outputs
  float2* part;   // [N][n_vtiles] (M, s)
  float* zt;      // [N] target logit
  float* logits;  // [N][ldz] fp32 logits, written by the storing forward only
  int64_t ldz;
  // backward inputs / output
  const float* lse;
  const float* grad;
  float* dl;
  int64_t ldg;
};

// Forward epilogue of token column j of a wave's block column: the (M, s)
// partial of the column's logits over the wave's 128 vocabulary rows -- the
// lane's maximum, then its sum of exponentials in (i, e) order, then the two
// lane halves merged -- and, where the column's target falls in these rows,
// the target's fp32 logit written to zt[tok].  A full vocabulary tile (the
// common case, a uniform branch) needs no row test; a ragged last tile skips
// its rows past V.  Every forward kernel forms its partials here, so a
// token's partial does not depend on which of them computed its tile.
template <int j, int NJ>
__device__ __forceinline__ float2 column_partial(const f32x16_t (&acc)[kI][NJ], int wv,
                                                 int half, int V_tail, bool have, int64_t t,
                                                 int vwave, float* zt, int64_t tok) {
  float mx = neg_inf();
  float M = neg_inf();
  float s = 0.0f;
  if (V_tail >= kBV) {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = vmax(mx, acc[i][j][e]);
    const float Mu = lse_raise(M, s, mx);
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) s = s + lse_term(acc[i][j][e], Mu);
  } else {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = wv * 128 + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < V_tail) mx = vmax(mx, acc[i][j][e]);
      }
    const float Mu = lse_raise(M, s, mx);
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = wv * 128 + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < V_tail) s = s + lse_term(acc[i][j][e], Mu);
      }
  }
  if (have) {
    const int64_t d = t - vwave;
    if (d >= 0 && d < 128) {
      const int dd = static_cast<int>(d);
      const int rem = dd & 31;
      if (((rem >> 2) & 1) == half) {
        // vocabulary row dd of this wave = block dd >> 5, element
        // 4 ((dd & 31) >> 3) + (dd & 3)
        const int idx = 16 * (dd >> 5) + (((rem >> 3) << 2) | (rem & 3));
        zt[tok] = select_acc(acc, j, idx);
      }
    }
  }
  const float M2 = __shfl_xor(M, 32, 64);
  const float s2 = __shfl_xor(s, 32, 64);
  lse_merge(M, s, M2, s2);
  return make_float2(M, s);
}

// Per-token terms of the dlogits epilogue for token column tok of a lane
// whose first vocabulary row is vlane (vwave + 4 * half).  d = g ([v == t] -
// p) is formed without branches: p is always evaluated, a masked row (or a
// token column past N) selects +0 whatever its logits hold, an active row
// with an invalid target carries NaN in the additive term, and NaN or
// infinite logits of an active row reach its gradient unclamped.
struct DlogitsColumn {
  bool active;
  float g;
  float ng;
  float off;     // lse * log2(e)
  float poison;  // NaN for an active row with an invalid target, else +0
  int rel;       // the target's offset from vlane, or -1 when outside [0, 128)
};

__device__ __forceinline__ DlogitsColumn dlogits_column(const TileArgs& args, bool have,
                                                        int64_t tok, int vlane) {
  DlogitsColumn c;
  c.active = have && ((args.mask == nullptr) || (args.mask[tok] != 0));
  const int64_t t = c.active ? args.targets[tok] : -1;
  const bool tvalid = (t >= 0 && t < args.V);
  c.g = c.active ? args.grad[tok] : 0.0f;
  c.ng = -c.g;
  c.off = c.active ? args.lse[tok] * kLog2e : 0.0f;
  const int64_t rt = t - vlane;
  c.rel = (rt >= 0 && rt < 128) ? static_cast<int>(rt) : -1;
  c.poison = (c.active && !tvalid) ? __builtin_nanf("") : 0.0f;
  return c;
}

// dlogits of accumulator elements 4q .. 4q + 3 of block i, that is vocabulary
// rows vlane + 32 i + 8 q + e, e = 0 .. 3.
__device__ __forceinline__ float4 dlogits_quad(const f32x16_t& a, int i, int q,
                                               const DlogitsColumn& c) {
  float d[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = fast_exp2(__builtin_fmaf(a[4 * q + e], kLog2e, -c.off));
    const float add = (i * 32 + 8 * q + e == c.rel) ? c.g : 0.0f;
    d[e] = c.active ? __builtin_fmaf(c.ng, p, add + c.poison) : 0.0f;
  }
  return make_float4(d[0], d[1], d[2], d[3]);
}

// blockIdx -> (vocabulary tile, token block): XCD-contiguous ranges, then
// groups of kLinearVocabGroup vocabulary tiles x all token blocks.
__device__ __forceinline__ void tile_coords(int w, int n_vtiles, int n_tblocks, int& vt, int& tb) {
  grouped_coords(w, n_vtiles, n_tblocks, kLinearVocabGroup, vt, tb);
}

// Backward tile kernel: the forward's per-tile main loop (same copies, same
// MFMA sequence, hence bit-identical logits), then the dlogits epilogue.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_tiles_bwd(TileArgs args) {
  __shared__ uint4 smem[kSmemVec];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave / kWQ;  // vocabulary half of the tile
  const int wt = wave % kWQ;  // token quarter of the tile
  int vt, tb;
  tile_coords(blockIdx.x, args.n_vtiles, args.n_tblocks, vt, tb);
  const int vocab0 = vt * kBV;
  const int64_t tok0 = static_cast<int64_t>(tb) * kBT;
  const int N_tail = static_cast<int>(min<int64_t>(args.N - tok0, kBT));  // rows of this block < N
  const int V_tail = min(args.V - vocab0, kBV);

  // W rows past V and hidden rows past N lie outside the resources' ranges
  // and read as zero.
  const __amdgpu_buffer_rsrc_t wres =
      uniform_rsrc(args.weight + static_cast<int64_t>(vocab0) * args.ldw, V_tail * args.ldw * 2);
  const __amdgpu_buffer_rsrc_t hres = uniform_rsrc(args.hidden + tok0 * args.ldh, N_tail * args.ldh * 2);
  const Loader ld = make_loader(wave, lane, args.ldw, args.ldh);
  f32x16_t acc[kI][kJ];
  mainloop(smem, ld, wave, lane, wv, wt, wres, hres, args.H, acc);

  // Result layout of a 32x32 MFMA block: lane holds token column
  // (lane & 31) and vocabulary rows 8 (e >> 2) + 4 (lane >> 5) + (e & 3).
  const int half = lane >> 5;
  const int vwave = vocab0 + wv * 128;  // first vocabulary entry of this wave

  {
    // dlogits tile, staged through LDS one 32-token slice at a time so that
    // each store instruction writes two 512-byte row segments.
    float* stage = reinterpret_cast<float*>(smem) + wave * (32 * kStageStride);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int tl = wt * kQW + j * 32 + (lane & 31);
      const DlogitsColumn c = dlogits_column(args, tl < N_tail, tok0 + tl, vwave + 4 * half);
      float* srow = stage + (lane & 31) * kStageStride;
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(srow + i * 32 + 8 * q + 4 * half) = dlogits_quad(acc[i][j], i, q, c);
      __syncthreads();
#pragma unroll 4
      for (int step = 0; step < 16; ++step) {
        const int r = 2 * step + (lane >> 5);
        const int c4 = lane & 31;
        const int tr = wt * kQW + j * 32 + r;
        if (tr < N_tail) {
          const float4 v = *reinterpret_cast<const float4*>(stage + r * kStageStride + 4 * c4);
          const int mrel = wv * 128 + 4 * c4;  // relative to vocab0
          float* dst = args.dl + (tok0 + tr) * args.ldg + vocab0 + mrel;
          if (mrel + 4 <= V_tail) {
            store16_stream(dst, v.x, v.y, v.z, v.w);
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mrel + e < V_tail) dst[e] = vv[e];
          }
        }
      }
      __syncthreads();
    }
  }
}

// Forward: one workgroup per tile, the tile core's main loop (the same copies
// and MFMA sequence in the same K order as linear_tiles_bwd, so the backward
// recomputes the very same logits), then the epilogue: per token, the (M, s)
// partial of the tile's 256 logits (lane-local in (i, e) order, then the two
// lane halves, then the two vocabulary waves through LDS) and, where the
// target falls in the tile, its fp32 logit.  With kStoreLogits the epilogue
// also writes the tile's fp32 logits (every row below N, every column below
// V), staged through the LDS as the backward stages its gradient.
template <bool kStoreLogits>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_tiles_fwd(TileArgs args) {
  // the storing variant stages its logits through the LDS like the backward
  __shared__ uint4 smem[kStoreLogits ? kSmemVec : 2 * kStageVec];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave / kWQ;
  const int wt = wave % kWQ;
  struct Geo {
    int vt;
    int vocab0;
    int64_t tok0;
    int V_tail;  // vocabulary entries of this tile below V
    int N_tail;  // token rows of this tile below N
  } cur;
  int tb;
  tile_coords(blockIdx.x, args.n_vtiles, args.n_tblocks, cur.vt, tb);
  cur.vocab0 = cur.vt * kBV;
  cur.tok0 = static_cast<int64_t>(tb) * kBT;
  cur.N_tail = static_cast<int>(min<int64_t>(args.N - cur.tok0, kBT));
  cur.V_tail = min(args.V - cur.vocab0, kBV);
  // targets of this lane's token columns, loaded before the main loop's
  // copies so that waiting for them never waits for a copy
  int64_t tgt[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int tl = wt * kQW + j * 32 + (lane & 31);
    tgt[j] = (tl < cur.N_tail) ? args.targets[cur.tok0 + tl] : -1;
  }
  // W rows past V and hidden rows past N lie outside the resources' ranges
  // and read as zero.
  const __amdgpu_buffer_rsrc_t wres = uniform_rsrc(
      args.weight + static_cast<int64_t>(cur.vocab0) * args.ldw, cur.V_tail * args.ldw * 2);
  const __amdgpu_buffer_rsrc_t hres =
      uniform_rsrc(args.hidden + cur.tok0 * args.ldh, cur.N_tail * args.ldh * 2);
  const Loader ld = make_loader(wave, lane, args.ldw, args.ldh);
  f32x16_t acc[kI][kJ];
  mainloop(smem, ld, wave, lane, wv, wt, wres, hres, args.H, acc);

  const int half = lane >> 5;
  const int vwave = cur.vocab0 + wv * 128;
  // the main loop ended with a barrier: the whole LDS is free
  float2* red = reinterpret_cast<float2*>(smem);
  if constexpr (kStoreLogits) {
    // the logits tile, staged through LDS one 32-token slice at a time so
    // that each store instruction writes two 512-byte row segments (the main
    // loop ended with a barrier, so the LDS is free)
    float* stage = reinterpret_cast<float*>(smem) + wave * (32 * kStageStride);
    float* srow = stage + (lane & 31) * kStageStride;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m0 = i * 32 + 8 * q + 4 * half;  // relative to vwave
          *reinterpret_cast<float4*>(srow + m0) = make_float4(
              acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      __syncthreads();
#pragma unroll 4
      for (int step = 0; step < 16; ++step) {
        const int r = 2 * step + (lane >> 5);
        const int c4 = lane & 31;
        const int tr = wt * kQW + j * 32 + r;
        if (tr < cur.N_tail) {
          const float4 v = *reinterpret_cast<const float4*>(stage + r * kStageStride + 4 * c4);
          const int mrel = wv * 128 + 4 * c4;  // relative to vocab0
          float* dst = args.logits + (cur.tok0 + tr) * args.ldz + cur.vocab0 + mrel;
          if (mrel + 4 <= cur.V_tail) {
            store16_stream(dst, v.x, v.y, v.z, v.w);
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mrel + e < cur.V_tail) dst[e] = vv[e];
          }
        }
      }
      __syncthreads();
    }
  }
  // the column index is a template argument: with a run-time index the
  // accumulators would be addressed as an array in scratch memory
  static_assert(kJ == 2, "two token block columns per wave");
  {
    const int tl = wt * kQW + (lane & 31);
    const float2 ms = column_partial<0>(acc, wv, half, cur.V_tail, tl < cur.N_tail, tgt[0], vwave,
                                        args.zt, cur.tok0 + tl);
    if (half == 0) red[wv * kBT + tl] = ms;
  }
  {
    const int tl = wt * kQW + 32 + (lane & 31);
    const float2 ms = column_partial<1>(acc, wv, half, cur.V_tail, tl < cur.N_tail, tgt[1], vwave,
                                        args.zt, cur.tok0 + tl);
    if (half == 0) red[wv * kBT + tl] = ms;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (tid < kBT) {
    const int tl = tid;
    float2 p0 = red[tl];
    const float2 p1 = red[kBT + tl];
    lse_merge(p0.x, p0.y, p1.x, p1.y);
    if (tl < cur.N_tail) args.part[(cur.tok0 + tl) * args.n_vtiles + cur.vt] = p0;
  }
}

// Small batches (at most 128 token rows).  All rows lie in the first 32, 64
// or 128 token columns of a tile (NJ = 1, 2 or 4 blocks of 32), so of the
// tile's MFMA work only the blocks (i, j < NJ) matter, and the tile is bound
// by streaming its 256 W rows.  The small-batch kernels run exactly those
// blocks -- the same fragments, the same v_mfma_f32_32x32x16_bf16 sequence
// in the same K order, hence the same fp32 logits -- and the forward ends
// with the same column epilogue and wave merge (column_partial, then
// vocabulary half 0 before half 1), so every row's partials, z_t, logp and
// lse, and every dlogits entry of the backward, are bit-identical to those
// of the full tile kernels.  What differs is the launch: one workgroup of
// 2 NJ waves per 256-entry vocabulary tile, wave (wv, jw) owning the blocks
// (i, jw) of vocabulary half wv; W reaches the LDS through registers
// (16-byte buffer loads, eight lanes per 128-byte row segment, the next
// stage's loads in flight while this stage is consumed) instead of
// direct-to-LDS copies, which stream this pattern about a sixth slower; and
// the LDS holds one stage of W and of the batch's hidden rows (36, 40 or
// 48 KB), so four, three or two workgroups fit on a compute unit and a
// vocabulary of up to 1024, 768 or 512 tiles streams in a single round.
constexpr int kAuxNontemporal = 2;  // cache-policy bits of a buffer load: nt

template <int NJ>
struct SmallGeo {
  static constexpr int kWaves = 2 * NJ;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * NJ;                  // token rows held
  static constexpr int kWVec = kBV * kRowChunks;         // uint4 of W per stage (32 KB)
  static constexpr int kHVec = kRows * kRowChunks;       // uint4 of hidden per stage
  static constexpr int kStageVec = kWVec + kHVec;
  static constexpr int kWLoads = kWVec / 64 / kWaves;    // 16-byte loads per lane and stage
  static constexpr int kHLoads = kHVec / 64 / kWaves;
  static constexpr int kPerCU = NJ == 1 ? 4 : (NJ == 2 ? 3 : 2);  // workgroups per CU
  static constexpr int kWavesPerSimd = kPerCU * kWaves / 4;
  static_assert(kPerCU * kStageVec * 16 <= 160 * 1024, "LDS of the resident workgroups");
  static_assert(kWLoads * 64 * kWaves == kWVec && kHLoads * 64 * kWaves == kHVec, "load split");
};

// One operand's part of a stage for this lane: chunk idx = (wave * n + q) *
// 64 + lane of the stage, that is row 8 (wave * n + q) + lane / 8, logical
// chunk lane % 8.  A buffer load whose resource ends after the operand's
// last present row (so rows past it read as zero); the lane's byte offset
// within its row group is fixed (voff), the row group and the K position go
// in the scalar offset.  Chunks at or past K are zeroed after the load.  W is
// read once (nontemporal); the hidden rows are read by every tile (cached).
template <int kAux, int NL>
__device__ __forceinline__ void small_load(uint4 (&v)[NL], __amdgpu_buffer_rsrc_t res, int voff,
                                           int group_bytes, int wave, int lane, int k0, int K) {
  const bool in_k = k0 + 8 * (lane & 7) < K;
  const int s0 = __builtin_amdgcn_readfirstlane(wave * NL * group_bytes + 2 * k0);
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(res, voff, s0 + q * group_bytes, kAux);
    v[q] = in_k ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// ... written to the stage's LDS rows at the tile layout's swizzled chunk.
template <int NL>
__device__ __forceinline__ void small_store(uint4* dst, const uint4 (&v)[NL], int wave, int lane) {
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int idx = (wave * NL + q) * 64 + lane;
    const int r = idx / kRowChunks;
    dst[r * kRowChunks + swz(r, idx % kRowChunks)] = v[q];
  }
}

// The small-batch main loop of wave (wv, jw): each stage of W and of the
// batch's hidden rows passes through registers into the tile layout in the
// LDS (the next stage's loads are issued right after), and the wave runs
// the blocks (i, jw) with the tile core's fragments and MFMA order.  Two
// barriers per stage: the stage is visible before its reads, and its reads
// end before the next stage overwrites it.  The LDS is free on return.
template <int NJ>
__device__ __forceinline__ void small_mainloop(uint4* smem, const TileArgs& args, int wave,
                                               int lane, int vocab0, int V_tail, int N,
                                               f32x16_t (&acc)[kI][1]) {
  using G = SmallGeo<NJ>;
  const int wv = wave & 1;
  const int jw = wave >> 1;
  // W rows past V and hidden rows past N lie outside the resources' ranges
  const __amdgpu_buffer_rsrc_t wres =
      uniform_rsrc(args.weight + static_cast<int64_t>(vocab0) * args.ldw, V_tail * args.ldw * 2);
  const __amdgpu_buffer_rsrc_t hres = uniform_rsrc(args.hidden, N * args.ldh * 2);
  const int wgrp = static_cast<int>(args.ldw) * 16;  // bytes of 8 rows
  const int hgrp = static_cast<int>(args.ldh) * 16;
  const int wvoff = (lane >> 3) * static_cast<int>(args.ldw) * 2 + 16 * (lane & 7);
  const int hvoff = (lane >> 3) * static_cast<int>(args.ldh) * 2 + 16 * (lane & 7);
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][0][e] = 0.0f;
  const int K = args.H;
  const int n_kt = (K + kBK - 1) / kBK;
  uint4 wr[G::kWLoads], hr[G::kHLoads];
  small_load<kAuxNontemporal>(wr, wres, wvoff, wgrp, wave, lane, 0, K);
  small_load<0>(hr, hres, hvoff, hgrp, wave, lane, 0, K);
  const uint4* a = smem;
  const uint4* b = smem + G::kWVec;
  for (int kt = 0; kt < n_kt; ++kt) {
    small_store(smem, wr, wave, lane);
    small_store(smem + G::kWVec, hr, wave, lane);
    if (kt + 1 < n_kt) {
      small_load<kAuxNontemporal>(wr, wres, wvoff, wgrp, wave, lane, (kt + 1) * kBK, K);
      small_load<0>(hr, hres, hvoff, hgrp, wave, lane, (kt + 1) * kBK, K);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSub; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8_t fa[kI];
#pragma unroll
      for (int i = 0; i < kI; ++i) {
        const int r = wv * kPW + i * 32 + (lane & 31);
        fa[i] = __builtin_bit_cast(bf16x8_t, a[r * kRowChunks + swz(r, c)]);
      }
      const int rq = jw * 32 + (lane & 31);
      const bf16x8_t fb = __builtin_bit_cast(bf16x8_t, b[rq * kRowChunks + swz(rq, c)]);
#pragma unroll
      for (int i = 0; i < kI; ++i)
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb, acc[i][0], 0, 0, 0);
    }
    __syncthreads();
  }
}

template <int NJ>
__global__ __launch_bounds__(SmallGeo<NJ>::kThreads)
__attribute__((amdgpu_waves_per_eu(SmallGeo<NJ>::kWavesPerSimd)))
void linear_tiles_fwd_small(TileArgs args) {
  using G = SmallGeo<NJ>;
  __shared__ uint4 smem[G::kStageVec];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave & 1;  // vocabulary half of the tile
  const int vt = blockIdx.x;
  const int vocab0 = vt * kBV;
  const int V_tail = min(args.V - vocab0, kBV);
  const int N = static_cast<int>(args.N);  // at most G::kRows
  const int tl = (wave >> 1) * 32 + (lane & 31);  // this lane's token row
  f32x16_t acc[kI][1];
  small_mainloop<NJ>(smem, args, wave, lane, vocab0, V_tail, N, acc);
  // (the target is read after the main loop: held across it, it would push
  // the 64-row form past its register budget)
  const int64_t tgt = (tl < N) ? args.targets[tl] : -1;

  const int half = lane >> 5;
  const int vwave = vocab0 + wv * kPW;
  float2* red = reinterpret_cast<float2*>(smem);
  const float2 ms = column_partial<0>(acc, wv, half, V_tail, tl < N, tgt, vwave, args.zt,
                                      static_cast<int64_t>(tl));
  if (half == 0) red[wv * G::kRows + tl] = ms;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (int r = tid; r < G::kRows; r += G::kThreads) {
    float2 p0 = red[r];
    const float2 p1 = red[G::kRows + r];
    lse_merge(p0.x, p0.y, p1.x, p1.y);
    if (r < N) args.part[static_cast<int64_t>(r) * args.n_vtiles + vt] = p0;
  }
}

// Backward for a small batch: the small-batch main loop (the same logits as
// linear_tiles_bwd's, bit for bit), then the dlogits of each wave's 128 x 32
// block (dlogits_quad, the same formula as the full tile's epilogue),
// staged through the LDS in two passes of 64 vocabulary rows so that each
// store instruction writes four 256-byte row segments.
constexpr int kSmallStageStride = 68;  // floats per staged token row (64 + 4 pad)

template <int NJ>
__global__ __launch_bounds__(SmallGeo<NJ>::kThreads)
__attribute__((amdgpu_waves_per_eu(SmallGeo<NJ>::kWavesPerSimd)))
void linear_tiles_bwd_small(TileArgs args) {
  using G = SmallGeo<NJ>;
  constexpr int kStagingVec = G::kWaves * 32 * kSmallStageStride / 4;
  constexpr int kSmemVec = G::kStageVec > kStagingVec ? G::kStageVec : kStagingVec;
  static_assert(G::kPerCU * kSmemVec * 16 <= 160 * 1024, "LDS of the resident workgroups");
  __shared__ uint4 smem[kSmemVec];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave & 1;  // vocabulary half of the tile
  const int jw = wave >> 1;  // token block of the wave
  const int vt = blockIdx.x;
  const int vocab0 = vt * kBV;
  const int V_tail = min(args.V - vocab0, kBV);
  const int N = static_cast<int>(args.N);  // at most G::kRows
  const int half = lane >> 5;
  const int vlane = vocab0 + wv * kPW + 4 * half;  // this lane's first vocabulary row
  const int tl = jw * 32 + (lane & 31);            // this lane's token row
  const DlogitsColumn col = dlogits_column(args, tl < N, tl, vlane);
  f32x16_t acc[kI][1];
  small_mainloop<NJ>(smem, args, wave, lane, vocab0, V_tail, N, acc);

  // the main loop ended with a barrier: the whole LDS is free
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * kSmallStageStride);
  float* srow = stage + (lane & 31) * kSmallStageStride;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // blocks 2p and 2p + 1: vocabulary rows wv * 128 + 64 p .. + 63
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(srow + ii * 32 + 8 * q + 4 * half) =
            dlogits_quad(acc[2 * p + ii][0], 2 * p + ii, q, col);
    __syncthreads();
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const int r = 4 * step + (lane >> 4);  // staged token row
      const int c4 = lane & 15;
      const int tr = jw * 32 + r;
      if (tr < N) {
        const float4 v = *reinterpret_cast<const float4*>(stage + r * kSmallStageStride + 4 * c4);
        const int m = wv * kPW + 64 * p + 4 * c4;  // relative to vocab0
        float* dst = args.dl + static_cast<int64_t>(tr) * args.ldg + vocab0 + m;
        if (m + 4 <= V_tail) {
          store16_stream(dst, v.x, v.y, v.z, v.w);
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m + e < V_tail) dst[e] = vv[e];
        }
      }
    }
    __syncthreads();
  }
}

// One wave per row: lane l merges the row's chunk partials l, l + 64,
// l + 128, ... in ascending order, then the 64 lane states merge in the fixed
// butterfly; the schedule depends on the number of chunks (that is, on V)
// only.  Partials are row-major, so each step is one coalesced 512-byte load.
// A launch of more rows than the grid holds loops (rows + gridDim.x * 4).
constexpr int kCombineRows = 4;  // rows (waves) per workgroup
constexpr int64_t kCombineMaxGrid = int64_t(1) << 22;

__global__ __launch_bounds__(64 * kCombineRows) void lse_chunk_combine(
    const float2* __restrict__ part, int n_vtiles, const float* __restrict__ zt,
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ mask, int64_t N, int V,
    float* __restrict__ logp, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kCombineRows + (threadIdx.x >> 6);
       row < N; row += static_cast<int64_t>(gridDim.x) * kCombineRows) {
  if (mask != nullptr && mask[row] == 0) {
    if (lane == 0) {
      logp[row] = 0.0f;
      if (lse != nullptr) lse[row] = 0.0f;
    }
    continue;
  }
  const float2* rp = part + row * n_vtiles;
  float M = neg_inf();
  float s = 0.0f;
  int c = lane;
  // four loads in flight per lane, merged in ascending chunk order
  for (; c + 192 < n_vtiles; c += 256) {
    const float2 p0 = rp[c];
    const float2 p1 = rp[c + 64];
    const float2 p2 = rp[c + 128];
    const float2 p3 = rp[c + 192];
    lse_merge(M, s, p0.x, p0.y);
    lse_merge(M, s, p1.x, p1.y);
    lse_merge(M, s, p2.x, p2.y);
    lse_merge(M, s, p3.x, p3.y);
  }
  for (; c < n_vtiles; c += 64) {
    const float2 p = rp[c];
    lse_merge(M, s, p.x, p.y);
  }
  wave_lse_allreduce(M, s, lane);
  if (lane == 0) {
    const float l = lse_finish(M, s);
    const int64_t t = targets[row];
    logp[row] = (t >= 0 && t < V) ? zt[row] - l : __builtin_nanf("");
    if (lse != nullptr) lse[row] = l;
  }
  }
}

TileArgs make_args(const uint16_t* hidden, int64_t ldh, const uint16_t* weight, int64_t ldw,
                   const int64_t* targets, const uint8_t* mask, int64_t N, int V, int H) {
  TileArgs a{};
  a.hidden = hidden;
  a.ldh = ldh;
  a.weight = weight;
  a.ldw = ldw;
  a.targets = targets;
  a.mask = mask;
  a.N = N;
  a.V = V;
  a.H = H;
  a.n_vtiles = (V + kBV - 1) / kBV;
  a.n_tblocks = static_cast<int>((N + kBT - 1) / kBT);
  return a;
}

}  // namespace

size_t linear_workspace_bytes(int64_t N, int64_t V) {
  const int64_t n_vtiles = (V + kBV - 1) / kBV;
  const size_t part = static_cast<size_t>(n_vtiles) * static_cast<size_t>(N) * sizeof(float2);
  const size_t zt = static_cast<size_t>(N) * sizeof(float);
  const size_t bytes = ((part + 255) / 256) * 256 + ((zt + 255) / 256) * 256;
  return bytes;
}

hipError_t launch_linear_logp(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                              int64_t ldw, const int64_t* targets, const uint8_t* mask, int64_t N,
                              int V, int H, float* logp, float* lse, float* logits, int64_t ldz,
                              void* workspace, hipStream_t stream) {
  TileArgs a = make_args(hidden, ldh, weight, ldw, targets, mask, N, V, H);
  const int64_t n_vtiles = a.n_vtiles;
  const size_t part_bytes = ((static_cast<size_t>(n_vtiles) * N * sizeof(float2) + 255) / 256) * 256;
  a.part = reinterpret_cast<float2*>(workspace);
  a.zt = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + part_bytes);
  a.logits = logits;
  a.ldz = ldz;
  const uint32_t tiles = static_cast<uint32_t>(static_cast<int64_t>(a.n_vtiles) * a.n_tblocks);
  if (logits != nullptr)
    hipLaunchKernelGGL(linear_tiles_fwd<true>, dim3(tiles), dim3(kThreads), 0, stream, a);
  else if (N <= SmallGeo<1>::kRows)
    hipLaunchKernelGGL(linear_tiles_fwd_small<1>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<1>::kThreads), 0, stream, a);
  else if (N <= SmallGeo<2>::kRows)
    hipLaunchKernelGGL(linear_tiles_fwd_small<2>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<2>::kThreads), 0, stream, a);
  else if (N <= SmallGeo<4>::kRows)
    hipLaunchKernelGGL(linear_tiles_fwd_small<4>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<4>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(linear_tiles_fwd<false>, dim3(tiles), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cgrid = (N + kCombineRows - 1) / kCombineRows;
  hipLaunchKernelGGL(lse_chunk_combine,
                     dim3(static_cast<uint32_t>(cgrid < kCombineMaxGrid ? cgrid : kCombineMaxGrid)),
                     dim3(64 * kCombineRows), 0,
                     stream, a.part, a.n_vtiles, a.zt, targets, mask, N, V, logp, lse);
  return hipGetLastError();
}

hipError_t launch_linear_dlogits(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                                 int64_t ldw, const int64_t* targets, const uint8_t* mask,
                                 const float* lse, const float* grad, int64_t N, int V, int H,
                                 float* dl, int64_t ldg, hipStream_t stream) {
  TileArgs a = make_args(hidden, ldh, weight, ldw, targets, mask, N, V, H);
  a.lse = lse;
  a.grad = grad;
  a.dl = dl;
  a.ldg = ldg;
  const int64_t tiles = static_cast<int64_t>(a.n_vtiles) * a.n_tblocks;
  if (N <= SmallGeo<1>::kRows)
    hipLaunchKernelGGL(linear_tiles_bwd_small<1>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<1>::kThreads), 0, stream, a);
  else if (N <= SmallGeo<2>::kRows)
    hipLaunchKernelGGL(linear_tiles_bwd_small<2>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<2>::kThreads), 0, stream, a);
  else if (N <= SmallGeo<4>::kRows)
    hipLaunchKernelGGL(linear_tiles_bwd_small<4>, dim3(static_cast<uint32_t>(a.n_vtiles)),
                       dim3(SmallGeo<4>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(linear_tiles_bwd, dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace rlk
