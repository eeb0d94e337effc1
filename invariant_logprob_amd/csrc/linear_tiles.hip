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
// Tile = 256 vocabulary entries x 256 tokens, 4 waves as 2 (vocab) x 2
// (tokens), each wave 128 x 128 = 4 x 4 MFMA blocks.  A 256-wide vocabulary
// tile is also the reduction chunk: per token, the tile's 256 logits are
// reduced in a fixed order (lane-local ascending, then the two lane halves,
// then the two vocabulary waves) to one (M, s) partial, written to the
// workspace.  A second kernel merges a row's partials in ascending chunk
// order.  Rows beyond N in the last token block are zero-filled and never
// written.  The logits stay fp32 and are never rounded to bf16.
//
// The pages fix the contract these kernels keep: bitwise batch invariance
// (page "[RFC] Batch-Invariant RL Kernel Suite for Train-Inference
// Consistency", maintainer reply, relation I); fixed, shape-independent
// reduction order and no atomics (page "[WS1 Test] #154 dtype pin + ...",
// section "Workstream 3 - #153", scope item 2); bf16 inputs with fp32
// accumulation (same page, "Workstream 1 - #154" scope table).  The tile
// schedule, the MFMA instruction and the K order never depend on N.
//
// The backward kernel reruns exactly the forward's main loop (same template,
// same instruction sequence), so its z is bit-identical to the forward's, and
// replaces the epilogue by d = g (onehot - 2^(z log2 e - lse log2 e)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"

namespace rlk {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBV = kLinearVocabTile;   // vocabulary entries per tile (= chunk)
constexpr int kBT = kLinearTokenTile;   // tokens per tile
constexpr int kBK = kLinearKStage;      // K per pipeline stage
constexpr int kThreads = 256;
constexpr int kRowChunks = kBK / 8;     // 16-byte chunks per tile row per stage
constexpr int kAVec = kBV * kRowChunks; // uint4 per stage, W side
constexpr int kBVec = kBT * kRowChunks; // uint4 per stage, hidden side
constexpr int kStageVec = kAVec + kBVec;
constexpr int kLoadsPerThread = kAVec / kThreads;   // 8
static_assert(kAVec == kBVec, "loader assumes square tiles");
static_assert(kRowChunks == 8, "swizzle assumes 8 chunks per row");
static_assert(kLoadsPerThread * 4 * 8 == kBV, "4 waves x 8 loads x 8 rows cover the tile");

// Word 3 of a raw buffer resource on gfx9-family parts (data format field)
constexpr int kBufferResourceWord3 = 0x00020000;
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

// A byte offset beyond any buffer range: such loads return zero.
constexpr int kOutOfRange = 0x7ffffff0;

// LDS chunk swizzle: chunk c of tile row r is stored at c ^ ((r >> 1) & 7) so
// that the 16-byte fragment reads of consecutive rows spread over all banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
// generic pointer into __shared__ memory -> LDS address space pointer
__device__ __forceinline__ lds_void_ptr to_lds(uint4* p) { return (lds_void_ptr)(p); }

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
  float2* part;   // [n_vtiles][N] (M, s)
  float* zt;      // [N] target logit
  // backward inputs / output
  const float* lse;
  const float* grad;
  float* dl;
  int64_t ldg;
};

// blockIdx -> (vocabulary tile, token block).  Workgroups are dispatched
// round-robin over the 8 XCDs, so ids are first regrouped into contiguous
// per-XCD ranges; within a range, tiles are ordered by groups of
// kLinearVocabGroup vocabulary tiles x all token blocks, so the workgroups
// sharing an XCD (and its L2) work on few W tiles and few hidden blocks at a
// time.  A bijection on [0, n_tiles); it only decides *when* a tile runs,
// never how it is computed.
__device__ __forceinline__ void tile_coords(int w, int n_vtiles, int n_tblocks, int& vt, int& tb) {
  const int total = n_vtiles * n_tblocks;
  const int t8 = (total / 8) * 8;
  int L = w;
  if (w < t8) L = (w & 7) * (t8 / 8) + (w >> 3);
  const int span = kLinearVocabGroup * n_tblocks;
  const int g = L / span;
  const int rem = L - g * span;
  const int gsize = min(kLinearVocabGroup, n_vtiles - g * kLinearVocabGroup);
  tb = rem / gsize;
  vt = g * kLinearVocabGroup + (rem - tb * gsize);
}

template <bool kBackward>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void linear_tiles(TileArgs args) {
  __shared__ uint4 smem[2 * kStageVec];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave >> 1;  // vocabulary half of the tile
  const int wt = wave & 1;   // token half of the tile
  int vt, tb;
  tile_coords(blockIdx.x, args.n_vtiles, args.n_tblocks, vt, tb);
  const int vocab0 = vt * kBV;
  const int64_t tok0 = static_cast<int64_t>(tb) * kBT;
  const int N_tail = static_cast<int>(min<int64_t>(args.N - tok0, kBT));  // rows of this block < N
  const int V_tail = min(args.V - vocab0, kBV);
  const int H = args.H;
  const int n_kt = (H + kBK - 1) / kBK;

  // Loader: global -> LDS directly (buffer_load ... lds), no staging
  // registers.  Each wave instruction fills 1 KB of LDS = 8 tile rows of 128
  // bytes; lane l writes physical chunk (l & 7) of row 8 q + (l >> 3), which
  // holds logical chunk (l & 7) ^ swizzle(row).  Rows past V (or N) fall
  // outside the buffer's range and read as zero; chunks past H are forced
  // out of range the same way.
  const __amdgpu_buffer_rsrc_t wres =
      uniform_rsrc(args.weight + static_cast<int64_t>(vocab0) * args.ldw, V_tail * args.ldw * 2);
  const __amdgpu_buffer_rsrc_t hres = uniform_rsrc(args.hidden + tok0 * args.ldh, N_tail * args.ldh * 2);
  const int lrow = lane >> 3;   // row within an 8-row block
  const int lpc = lane & 7;     // physical chunk this lane fills

  auto issue = [&](int kt, int st) {
    const int k0 = kt * kBK;
    uint4* a = smem + st * kStageVec;
    uint4* b = a + kAVec;
#pragma unroll
    for (int q = 0; q < kLoadsPerThread; ++q) {
      const int blk = wave * kLoadsPerThread + q;     // 8-row block of the tile
      const int r = blk * 8 + lrow;
      const int c = lpc ^ ((r >> 1) & 7);
      const int k = k0 + 8 * c;
      const int woff = (k < H) ? (r * static_cast<int>(args.ldw) + k) * 2 : kOutOfRange;
      const int hoff = (k < H) ? (r * static_cast<int>(args.ldh) + k) * 2 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres, to_lds(a + blk * 64), 16, woff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          hres, to_lds(b + blk * 64), 16, hoff, 0, 0, 0);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](int st) {
    const uint4* a = smem + st * kStageVec;
    const uint4* b = a + kAVec;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wv * 128 + i * 32 + (lane & 31);
        fa[i] = __builtin_bit_cast(bf16x8_t, a[r * kRowChunks + swz(r, c)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wt * 128 + j * 32 + (lane & 31);
        fb[j] = __builtin_bit_cast(bf16x8_t, b[r * kRowChunks + swz(r, c)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // main loop: K stages in ascending order, two LDS buffers; the next
  // stage's loads are in flight while the current stage is multiplied
  issue(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // stage kt has landed; everyone is done with the other buffer
    if (kt + 1 < n_kt) issue(kt + 1, (kt + 1) & 1);
    compute(kt & 1);
  }
  __syncthreads();

  // Result layout of a 32x32 MFMA block: lane holds token column
  // (lane & 31) and vocabulary rows 8 (e >> 2) + 4 (lane >> 5) + (e & 3).
  const int half = lane >> 5;
  const int vwave = vocab0 + wv * 128;  // first vocabulary entry of this wave

  if constexpr (!kBackward) {
    float2* red = reinterpret_cast<float2*>(smem);  // [2][kBT], after the loop's last barrier
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wt * 128 + j * 32 + (lane & 31);
      const int64_t tok = tok0 + tl;
      float mx = neg_inf();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wv * 128 + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
          if (m < V_tail) mx = fmaxf(mx, acc[i][j][e]);
        }
      float M = neg_inf();
      float s = 0.0f;
      const float Mu = lse_raise(M, s, mx);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wv * 128 + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
          if (m < V_tail) {
#pragma clang fp contract(off)
            s = s + lse_term(acc[i][j][e], Mu);
          }
        }
      if (tl < N_tail) {
        const int64_t t = args.targets[tok];
        const int64_t d = t - vwave;
        if (d >= 0 && d < 128) {
          const int dd = static_cast<int>(d);
          const int rem = dd & 31;
          if (((rem >> 2) & 1) == half) {
            const int it = dd >> 5;
            const int et = ((rem >> 3) << 2) | (rem & 3);
            float val = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (i == it && e == et) val = acc[i][j][e];
            args.zt[tok] = val;
          }
        }
      }
      const float M2 = __shfl_xor(M, 32, 64);
      const float s2 = __shfl_xor(s, 32, 64);
      lse_merge(M, s, M2, s2);
      if (half == 0) red[wv * kBT + tl] = make_float2(M, s);
    }
    __syncthreads();
    {
      const int tl = tid;  // kThreads == kBT
      float2 p0 = red[tl];
      const float2 p1 = red[kBT + tl];
      lse_merge(p0.x, p0.y, p1.x, p1.y);
      if (tl < N_tail) args.part[static_cast<int64_t>(vt) * args.N + tok0 + tl] = p0;
    }
  } else {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wt * 128 + j * 32 + (lane & 31);
      if (tl >= N_tail) continue;
      const int64_t tok = tok0 + tl;
      const bool active = (args.mask == nullptr) || (args.mask[tok] != 0);
      const int64_t t = args.targets[tok];
      const bool tvalid = (t >= 0 && t < args.V);
      const float g = active ? args.grad[tok] : 0.0f;
      const float ng = -g;
      const float off = active ? args.lse[tok] * kLog2e : 0.0f;
      float* outp = args.dl + tok * args.ldg + vwave;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m0 = i * 32 + 8 * q + 4 * half;  // relative to vwave
          float d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(__builtin_fmaf(acc[i][j][4 * q + e], kLog2e, -off));
            const float add = (static_cast<int64_t>(vwave + m0 + e) == t) ? g : 0.0f;
            d[e] = __builtin_fmaf(ng, p, add);
            if (!active) d[e] = 0.0f;
            else if (!tvalid) d[e] = nan;
          }
          const int mrel = wv * 128 + m0;  // relative to vocab0
          if (mrel + 4 <= V_tail) {
            store16_stream(outp + m0, d[0], d[1], d[2], d[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (mrel + e < V_tail) outp[m0 + e] = d[e];
          }
        }
    }
  }
}

// Per row: merge the chunk partials in ascending chunk order, then finish.
__global__ __launch_bounds__(256) void lse_chunk_combine(const float2* __restrict__ part,
                                                         int n_vtiles, const float* __restrict__ zt,
                                                         const int64_t* __restrict__ targets,
                                                         const uint8_t* __restrict__ mask,
                                                         int64_t N, int V, float* __restrict__ logp,
                                                         float* __restrict__ lse) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= N) return;
  if (mask != nullptr && mask[row] == 0) {
    logp[row] = 0.0f;
    if (lse != nullptr) lse[row] = 0.0f;
    return;
  }
  float M = neg_inf();
  float s = 0.0f;
  for (int c = 0; c < n_vtiles; ++c) {
    const float2 p = part[static_cast<int64_t>(c) * N + row];
    lse_merge(M, s, p.x, p.y);
  }
  const float l = lse_finish(M, s);
  const int64_t t = targets[row];
  logp[row] = (t >= 0 && t < V) ? zt[row] - l : __builtin_nanf("");
  if (lse != nullptr) lse[row] = l;
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
                              int V, int H, float* logp, float* lse, void* workspace,
                              hipStream_t stream) {
  TileArgs a = make_args(hidden, ldh, weight, ldw, targets, mask, N, V, H);
  const int64_t n_vtiles = a.n_vtiles;
  const size_t part_bytes = ((static_cast<size_t>(n_vtiles) * N * sizeof(float2) + 255) / 256) * 256;
  a.part = reinterpret_cast<float2*>(workspace);
  a.zt = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + part_bytes);
  const int64_t tiles = static_cast<int64_t>(a.n_vtiles) * a.n_tblocks;
  hipLaunchKernelGGL((linear_tiles<false>), dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_chunk_combine, dim3(static_cast<uint32_t>((N + 255) / 256)), dim3(256), 0,
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
  hipLaunchKernelGGL((linear_tiles<true>), dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rlk
