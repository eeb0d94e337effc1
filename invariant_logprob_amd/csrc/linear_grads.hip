// Parameter gradients of the fused lm_head + selected logprob (gfx950):
//
//   grad_hidden = D . W      [N, H]     grad_weight = D^T . h      [V, H]
//
// with D the gradient with respect to the logits z = h . W^T,
// D_ij = g_i ([j == t_i] - exp(z_ij - lse_i)) (zero rows for inactive
// tokens).  These are the textbook chain-rule products; the pages ask that
// gradients keep the batch-invariance contract and that parameter gradients
// be compared over the same complete set of samples (page "[WS1 Test] #154
// dtype pin + #152 KV path + #153 bwd invariance + #150 chain gate", section
// "Workstream 3 - #153").
//
// D is never materialised whole.  The vocabulary is walked in fixed chunks
// of kGradChunk entries (a constant: the chunking depends on V only).  Per
// chunk c, in ascending c on the caller's stream:
//   1. grad_dl_tiles recomputes the chunk's logits with the forward's tile
//      main loop (bit-identical z), forms D in fp32 exactly as the logits
//      backward does and writes it as two bf16 arrays, the MFMA operand type:
//      D_hi = D rounded to bf16 and D_lo = (D - D_hi) rounded to bf16.  D -
//      D_hi is exact in fp32, so D_hi + D_lo holds D to a relative 2^-16:
//      the products see fp32-grade D (bf16 inputs, fp32 accumulation) rather
//      than D rounded once to 8 significant bits.  Given the fp32 logits the
//      forward kept, grad_dl_from_logits forms the same pair from them,
//      element by element with the same arithmetic, so the gradients come
//      out bit-identical at a fraction of the cost.
//   2. grad_gemm_tiles runs both products of the chunk in one launch, each
//      as two passes over its K into the same fp32 accumulators, first with
//      D_hi, then with D_lo:
//      grad_hidden (+)= D_c . W_c   (K = the chunk's vocabulary, ascending;
//                                    chunk 0 writes, later chunks add)
//      grad_weight[c] = D_c^T . h   (K = tokens, ascending)
//      W_c, h and (for the second product) D_c are contracted over their
//      rows, so those operands are read in their natural K-major layout
//      through transposing LDS reads: nothing is transposed in memory.
//
// Invariance.  A row of grad_hidden depends on its own row of D and on W
// only, through a K order fixed by V: bit-identical for any batch.  A row of
// grad_weight sums over every token of the batch in ascending row order: it
// is deterministic run to run, but a different batch composition is a
// different sum (the pages compare parameter gradients only over the same
// complete sample set).  No atomics anywhere.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"
#include "tile_core.hpp"

namespace rlk {

namespace {

using namespace tile;

// LDS staging of a 256 x 256 bf16 tile: rows of 256 entries + 8 pad.
constexpr int kDlStride = kBP + 8;  // bf16 elements per staged row
constexpr int kDlStageVec = kBQ * kDlStride * 2 / 16;
constexpr int kDlSmemVec = (2 * kStageVec > kDlStageVec) ? 2 * kStageVec : kDlStageVec;
static_assert(kDlSmemVec * 16 <= 160 * 1024, "LDS budget of one CU");
static_assert((kDlStride * 2) % 16 == 0, "staged rows must stay 16-byte aligned");

// fp32 output staging of the GEMM epilogue: per wave 32 rows of 128 + 4.
constexpr int kOutStride = 132;
constexpr int kOutStageVec = kWaves * 32 * kOutStride / 4;
constexpr int kGemmSmemVec = (2 * kStageVec > kOutStageVec) ? 2 * kStageVec : kOutStageVec;
static_assert(kGemmSmemVec * 16 <= 160 * 1024, "LDS budget of one CU");

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
}

// The bf16 word of part `lo` of x: x rounded to bf16 (lo = false), or the
// rounding's remainder x - bf16(x), itself rounded to bf16 (lo = true).  The
// remainder is exact in fp32 (x and bf16(x) are within a factor of 2), so the
// two words sum to x within a relative 2^-16.  NaN gives NaN in both.
__device__ __forceinline__ uint32_t bf16_part(float x, bool lo) {
#pragma clang fp contract(off)
  const uint32_t hi = bf16_bits(x);
  return lo ? bf16_bits(x - __uint_as_float(hi << 16)) : hi;
}

struct DlArgs {
  const uint16_t* hidden;
  int64_t ldh;
  const uint16_t* weight;
  int64_t ldw;
  const int64_t* targets;
  const uint8_t* mask;
  const float* lse;
  const float* grad;
  int64_t N;
  int V;
  int H;
  int vt0;        // first vocabulary tile of the chunk
  int n_vt;       // vocabulary tiles in the chunk
  int n_tblocks;  // 256-token blocks
  uint16_t* d;    // [N][ldd] bf16 D_hi, chunk-local columns
  uint16_t* d_lo; // [N][ldd] bf16 D_lo
  int64_t ldd;
};

// D (as D_hi and D_lo) for one 256-vocabulary x 256-token tile of the chunk.
// The main loop is the forward's (same operands, same K order), so z is
// bit-identical to the logits the forward reduced; the fp32 D formula is the
// logits backward's.  Entries past V, rows past N and inactive rows are
// written as zero; an active row with an invalid target, or with non-finite
// logits, gets NaN.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grad_dl_tiles(DlArgs a) {
  __shared__ uint4 smem[kDlSmemVec];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave / kWQ;
  const int wt = wave % kWQ;
  int vtl, tb;
  grouped_coords(blockIdx.x, a.n_vt, a.n_tblocks, kLinearVocabGroup, vtl, tb);
  const int vocab0 = (a.vt0 + vtl) * kBP;
  const int64_t tok0 = static_cast<int64_t>(tb) * kBQ;
  const int N_tail = static_cast<int>(min<int64_t>(a.N - tok0, kBQ));
  const int V_tail = min(a.V - vocab0, kBP);

  const __amdgpu_buffer_rsrc_t wres =
      uniform_rsrc(a.weight + static_cast<int64_t>(vocab0) * a.ldw, V_tail * a.ldw * 2);
  const __amdgpu_buffer_rsrc_t hres = uniform_rsrc(a.hidden + tok0 * a.ldh, N_tail * a.ldh * 2);
  const Loader ld = make_loader(wave, lane, a.ldw, a.ldh);
  f32x16_t acc[kI][kJ];
  mainloop(smem, ld, wave, lane, wv, wt, wres, hres, a.H, acc);

  // Per token column (lane & 31) of MFMA block j: what D needs of the row.
  const int half = lane >> 5;
  // rel[j]: the target's offset from this lane's first vocabulary row
  // (128 wv + 4 (lane >> 5) of the tile), or -1 when outside this wave's rows
  int rel[kJ];
  bool act[kJ];
  float ng[kJ], gg[kJ], off[kJ], pz[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int tl = wt * kQW + j * 32 + (lane & 31);
    const int64_t tok = tok0 + tl;
    const bool active = (tl < N_tail) && ((a.mask == nullptr) || (a.mask[tok] != 0));
    const int64_t t = active ? a.targets[tok] : -1;
    const bool tvalid = (t >= 0 && t < a.V);
    const int64_t r = t - (vocab0 + wv * 128 + 4 * half);
    rel[j] = (r >= 0 && r < 128) ? static_cast<int>(r) : -1;
    act[j] = active;
    gg[j] = active ? a.grad[tok] : 0.0f;
    ng[j] = -gg[j];
    off[j] = active ? a.lse[tok] * kLog2e : 0.0f;
    pz[j] = (active && !tvalid) ? __builtin_nanf("") : 0.0f;
  }
  // D of every accumulator entry is formed once and split into its two bf16
  // parts, both staged in LDS, one 32-token column block j of every wave at a
  // time (128 tokens x 256 vocabulary rows x 2 parts), then stored as whole
  // 512-byte token rows of D_hi and D_lo.  No branches: p is always
  // evaluated; a masked row or a column past V gets +0 whatever its logits
  // hold, an active row with an invalid target carries NaN in the additive
  // term, and NaN or infinite logits of an active row reach D unclamped.
  // kFull: the tile's 256 vocabulary rows are all < V (every tile but a
  // ragged last one), so no row test is needed -- a uniform branch picks it.
  auto epilogue = [&](auto full) {
  constexpr bool kFull = decltype(full)::value;
  uint16_t* S = reinterpret_cast<uint16_t*>(smem);
  constexpr int kHalfRows = kWQ * 32;                        // staged tokens per block j
  constexpr int kPieces = 2 * kHalfRows * (kBP / 8) / kThreads;  // 16-byte pieces per thread
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int sr = wt * 32 + (lane & 31);  // staged row of this lane's token
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int mrel = i * 32 + 8 * q + e;  // + 128 wv + 4 half
          const float p = fast_exp2(__builtin_fmaf(acc[i][j][4 * q + e], kLog2e, -off[j]));
          const float add = (mrel == rel[j]) ? gg[j] : 0.0f;
          const bool keep = act[j] && (kFull || wv * 128 + mrel + 4 * half < V_tail);
          // +0 for a dropped entry as a bit mask, not a select: a select lets
          // the compiler move the exponential under a branch per entry
          const float dv = __uint_as_float(
              __float_as_uint(__builtin_fmaf(ng[j], p, add + pz[j])) & (keep ? 0xffffffffu : 0u));
          hb[e] = bf16_part(dv, false);
          lb[e] = bf16_part(dv, true);
        }
        const int m0 = wv * 128 + i * 32 + 8 * q + 4 * half;
        *reinterpret_cast<uint2*>(S + sr * kDlStride + m0) =
            make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2*>(S + (kHalfRows + sr) * kDlStride + m0) =
            make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
      }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < kPieces; ++it) {
      const int idx = it * kThreads + tid;
      const int srow = idx >> 5;             // staged row: part * 128 + row
      const int c = idx & 31;
      const int r = srow & (kHalfRows - 1);
      const int tl = (r >> 5) * kQW + j * 32 + (r & 31);  // token within the tile
      if (tl < N_tail) {
        uint16_t* dst = (srow >= kHalfRows) ? a.d_lo : a.d;
        const uint4 v = *reinterpret_cast<const uint4*>(S + srow * kDlStride + 8 * c);
        *reinterpret_cast<uint4*>(dst + (tok0 + tl) * a.ldd + vtl * kBP + 8 * c) = v;
      }
    }
    __syncthreads();
  }
  };
  if (V_tail >= kBP) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// D_c (D_hi and D_lo) from kept fp32 logits [N, ldz]: entry (row, k) of the
// chunk is vocabulary column vocab0 + k.  The per-element arithmetic is
// grad_dl_tiles' (so is the split into two bf16 parts); columns at or past V
// within the padded chunk width and inactive rows get +0, and an active row
// with an invalid target NaN.  Blocks of 2048 columns of one row: 128 threads
// x 4 groups of 4 columns, 16-byte loads, 8-byte stores (512 contiguous bytes
// per wave instruction).
constexpr int kDlzThreads = 128;
constexpr int kDlzUnroll = 4;
constexpr int kDlzBlockCols = kDlzThreads * kDlzUnroll * 4;

__global__ __launch_bounds__(kDlzThreads) void grad_dl_from_logits(
    const float* __restrict__ logits, int64_t ldz, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, const float* __restrict__ lse,
    const float* __restrict__ grad, int64_t N, int V, int vocab0, int width, int nb,
    uint16_t* __restrict__ d, uint16_t* __restrict__ d_lo, int64_t ldd) {
  const int tid = threadIdx.x;
  const int64_t total = N * nb;
  for (int64_t wid = blockIdx.x; wid < total; wid += gridDim.x) {
    const int64_t row = wid / nb;
    const int k0 = static_cast<int>(wid - row * nb) * kDlzBlockCols;
    const bool active = (mask == nullptr) || (mask[row] != 0);
    const int64_t t = active ? targets[row] : -1;
    const float g = active ? grad[row] : 0.0f;
    const float ng = -g;
    const float off = active ? lse[row] * kLog2e : 0.0f;
    const float pz = (active && !(t >= 0 && t < V)) ? __builtin_nanf("") : 0.0f;
    const float* zr = logits + row * ldz + vocab0;
    uint16_t* dr = d + row * ldd;
    uint16_t* dlr = d_lo + row * ldd;
    float4 w[kDlzUnroll];
#pragma unroll
    for (int u = 0; u < kDlzUnroll; ++u) {
      const int k = k0 + 4 * (u * kDlzThreads + tid);
      w[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active && k < width && vocab0 + k < V) {
        if (vocab0 + k + 4 <= V) {
          w[u] = *reinterpret_cast<const float4*>(zr + k);
        } else {
          float x[4] = {0.f, 0.f, 0.f, 0.f};
          for (int e = 0; vocab0 + k + e < V; ++e) x[e] = zr[k + e];
          w[u] = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDlzUnroll; ++u) {
      const int k = k0 + 4 * (u * kDlzThreads + tid);
      if (k >= width) break;
      const float x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      uint32_t b[4], c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(__builtin_fmaf(x[e], kLog2e, -off));
        const bool keep = active && vocab0 + k + e < V;
        const float add = (vocab0 + k + e == t) ? g : 0.0f;
        const float dv = keep ? __builtin_fmaf(ng, p, add + pz) : 0.0f;
        b[e] = bf16_part(dv, false);
        c[e] = bf16_part(dv, true);
      }
      *reinterpret_cast<uint2*>(dr + k) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      *reinterpret_cast<uint2*>(dlr + k) = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
    }
  }
}

// One product of a chunk: out[Q rows][P rows] (+)= Q . P^T over K.  Each
// side is either an operand with one row per tile row and K contiguous, or a
// K-major operand whose columns are the tile rows (see tile_core.hpp).
struct GemmOp {
  const uint16_t* p;  // P side (output columns)
  int64_t ldp;
  int P;              // tile rows of the P side present
  int kext_p;         // K-major P: K rows present
  const uint16_t* q;  // Q side (output rows): D_hi
  const uint16_t* q_lo;  // D_lo, the same layout: a second pass over K
  int64_t ldq;
  int Q;
  int kext_q;
  int K;
  int q_kmajor;       // 0: Q one row per output row (grad_hidden); 1: Q K-major (grad_weight)
  float* out;         // [Q][ldo] fp32
  int64_t ldo;
  int accumulate;     // out = out + acc instead of out = acc
  int n_ptiles;
  int n_qtiles;
  int first;          // first workgroup of this product (a multiple of 8)
};

struct GemmArgs {
  GemmOp op[2];
  int n_ops;
};

// Both products of a chunk in one launch.  Workgroups [op[0].first, ...)
// compute op 0's tiles and [op[1].first, ...) op 1's; ids in between are
// idle padding that keeps each product's first id a multiple of 8 (the XCD
// regrouping works on ids relative to it).  The hardware dispatches
// workgroups in id order as compute units free up, so the long tiles listed
// first are spread over the chip before the short ones fill the gaps.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grad_gemm_tiles(GemmArgs args) {
  __shared__ uint4 smem[kGemmSmemVec];
  const bool second = (args.n_ops > 1) && (static_cast<int>(blockIdx.x) >= args.op[1].first);
  const GemmOp& g = second ? args.op[1] : args.op[0];
  const int w = static_cast<int>(blockIdx.x) - g.first;
  if (w < 0 || w >= g.n_ptiles * g.n_qtiles) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wp = wave / kWQ;
  const int wq = wave % kWQ;
  int qt, pt;
  grouped_coords(w, g.n_qtiles, g.n_ptiles, kLinearVocabGroup, qt, pt);
  const int p0 = pt * kBP;
  const int q0 = qt * kBQ;
  const int P_tail = min(g.P - p0, kBP);
  const int Q_tail = min(g.Q - q0, kBQ);

  f32x16_t acc[kI][kJ];
  // P is K-major in both products (W_c over the vocabulary, h over tokens).
  // Two passes over K into the same accumulators: D_hi, then D_lo.
  const Side Ps{g.p + p0, g.ldp, g.kext_p, p0};
  if (g.q_kmajor) {
    const LoaderG<Lay::kCols, Lay::kCols> ld = make_loader_g<Lay::kCols, Lay::kCols>(wave, lane, g.ldp, g.ldq);
#pragma nounroll
    for (int part = 0; part < 2; ++part) {
      const Side Qs{(part ? g.q_lo : g.q) + q0, g.ldq, g.kext_q, q0};
      mainloop_g(smem, ld, wave, lane, wp, wq, Ps, Qs, g.K, acc, part == 0);
    }
  } else {
    const LoaderG<Lay::kCols, Lay::kRows> ld = make_loader_g<Lay::kCols, Lay::kRows>(wave, lane, g.ldp, g.ldq);
#pragma nounroll
    for (int part = 0; part < 2; ++part) {
      const Side Qs{(part ? g.q_lo : g.q) + static_cast<int64_t>(q0) * g.ldq, g.ldq, Q_tail, 0};
      mainloop_g(smem, ld, wave, lane, wp, wq, Ps, Qs, g.K, acc, part == 0);
    }
  }

  // Staged through LDS one 32-row slice at a time so that each store
  // instruction writes two 512-byte row segments.
  const int half = lane >> 5;
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * kOutStride);
  float* srow = stage + (lane & 31) * kOutStride;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m0 = i * 32 + 8 * q + 4 * half;
        *reinterpret_cast<float4*>(srow + m0) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    __syncthreads();
#pragma unroll 4
    for (int step = 0; step < 16; ++step) {
      const int r = 2 * step + (lane >> 5);
      const int c4 = lane & 31;
      const int rr = wq * kQW + j * 32 + r;  // output row within the tile
      if (rr < Q_tail) {
        float4 v = *reinterpret_cast<const float4*>(stage + r * kOutStride + 4 * c4);
        const int mrel = wp * kPW + 4 * c4;  // output column within the tile
        float* dst = g.out + static_cast<int64_t>(q0 + rr) * g.ldo + p0 + mrel;
        if (mrel + 4 <= P_tail) {
          if (g.accumulate) {
            const float4 o = *reinterpret_cast<const float4*>(dst);
            v = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
          }
          store16_stream(dst, v.x, v.y, v.z, v.w);
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (mrel + e < P_tail) dst[e] = g.accumulate ? dst[e] + vv[e] : vv[e];
        }
      }
    }
    __syncthreads();
  }
}

// out[r][c] = 0 for r < rows, c < cols (cols % 4 == 0, 16-byte aligned rows)
__global__ __launch_bounds__(256) void zero_rows_f32(float* __restrict__ out, int64_t ldo,
                                                     int64_t rows, int cols) {
  const int64_t quads = static_cast<int64_t>(cols / 4);
  const int64_t total = rows * quads;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < total;
       k += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = k / quads;
    const int64_t c = (k - r * quads) * 4;
    *reinterpret_cast<float4*>(out + r * ldo + c) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// dst[r][0, H) = src[r][0, H) for active rows, +0 for inactive ones
// (H % 8 == 0, 16-byte aligned rows).  An inactive token's D row is zero,
// but its hidden row may hold anything, and 0 x inf or 0 x NaN would still
// reach every entry of grad_weight through the product; with the row zeroed
// the inactive token adds exact zeros, as the definition (a sum over active
// tokens) has it.
__global__ __launch_bounds__(256) void active_rows_bf16(const uint16_t* __restrict__ src,
                                                        int64_t lds, const uint8_t* __restrict__ mask,
                                                        int64_t rows, int cols,
                                                        uint16_t* __restrict__ dst, int64_t ldd) {
  const int64_t vecs = static_cast<int64_t>(cols / 8);
  const int64_t total = rows * vecs;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < total;
       k += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = k / vecs;
    const int64_t c = (k - r * vecs) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (mask[r] != 0) v = *reinterpret_cast<const uint4*>(src + r * lds + c);
    *reinterpret_cast<uint4*>(dst + r * ldd + c) = v;
  }
}

// Workspace: one chunk of D as two bf16 arrays, D_hi [N, chunk] and D_lo
// [N, chunk], then (used when a mask is given) a copy of hidden, [N, H] bf16,
// with inactive rows zeroed.
int64_t grad_d_bytes(int64_t N, int64_t V) {
  const int64_t chunk = min64(kGradChunk, round_up(V, kBP));
  return round_up(N * chunk * 2, 256);
}

size_t grad_workspace(int64_t N, int64_t V, int64_t H) {
  return static_cast<size_t>(2 * grad_d_bytes(N, V) + round_up(N * H * 2, 256));
}

}  // namespace

size_t linear_param_grads_workspace_bytes(int64_t N, int64_t V, int64_t H) {
  return grad_workspace(N, V, H);
}

hipError_t launch_linear_param_grads(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                                     int64_t ldw, const int64_t* targets, const uint8_t* mask,
                                     const float* lse, const float* grad, int64_t N, int V, int H,
                                     float* grad_hidden, int64_t ld_gh, float* grad_weight,
                                     int64_t ld_gw, const float* logits, int64_t ldz,
                                     void* workspace, hipStream_t stream) {
  if (N == 0) {
    // no tokens: grad_weight is an empty sum; grad_hidden has no rows
    if (grad_weight != nullptr) {
      const int64_t quads = static_cast<int64_t>(V) * (H / 4);
      const int64_t blocks = min64((quads + 255) / 256, 65536);
      hipLaunchKernelGGL(zero_rows_f32, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                         grad_weight, ld_gw, static_cast<int64_t>(V), H);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  uint16_t* d = static_cast<uint16_t*>(workspace);
  uint16_t* d_lo = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + grad_d_bytes(N, V));
  const int64_t chunk = min64(kGradChunk, round_up(V, kBP));
  const bool want_h = grad_hidden != nullptr;
  const bool want_w = grad_weight != nullptr;
  // grad_weight's token operand: hidden itself, or with a mask a copy whose
  // inactive rows are zero (made once for all chunks)
  const uint16_t* hw = hidden;
  int64_t ldhw = ldh;
  if (want_w && mask != nullptr) {
    uint16_t* hcopy = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                                  2 * grad_d_bytes(N, V));
    const int64_t vecs = N * (H / 8);
    const int64_t blocks = min64((vecs + 255) / 256, 65536);
    hipLaunchKernelGGL(active_rows_bf16, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       hidden, ldh, mask, N, H, hcopy, static_cast<int64_t>(H));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hw = hcopy;
    ldhw = H;
  }
  const int n_vtiles = (V + kBP - 1) / kBP;
  const int n_tblocks = static_cast<int>((N + kBQ - 1) / kBQ);
  const int tiles_per_chunk = static_cast<int>(chunk / kBP);
  const int n_chunks = (n_vtiles + tiles_per_chunk - 1) / tiles_per_chunk;
  const int n_htiles = (H + kBP - 1) / kBP;

  for (int c = 0; c < n_chunks; ++c) {
    const int vt0 = c * tiles_per_chunk;
    const int n_vt = static_cast<int>(min64(tiles_per_chunk, n_vtiles - vt0));
    const int vocab0 = vt0 * kBP;
    const int v_rows = static_cast<int>(min64(V - vocab0, n_vt * kBP));  // real vocabulary rows
    const int width = n_vt * kBP;                                        // padded chunk width

    if (logits != nullptr) {
      const int nb = (width + kDlzBlockCols - 1) / kDlzBlockCols;
      const int64_t blocks = min64(N * nb, int64_t(1) << 22);
      hipLaunchKernelGGL(grad_dl_from_logits, dim3(static_cast<uint32_t>(blocks)),
                         dim3(kDlzThreads), 0, stream, logits, ldz, targets, mask, lse, grad, N, V,
                         vocab0, width, nb, d, d_lo, static_cast<int64_t>(chunk));
    } else {
      DlArgs da{};
      da.hidden = hidden;
      da.ldh = ldh;
      da.weight = weight;
      da.ldw = ldw;
      da.targets = targets;
      da.mask = mask;
      da.lse = lse;
      da.grad = grad;
      da.N = N;
      da.V = V;
      da.H = H;
      da.vt0 = vt0;
      da.n_vt = n_vt;
      da.n_tblocks = n_tblocks;
      da.d = d;
      da.d_lo = d_lo;
      da.ldd = chunk;
      hipLaunchKernelGGL(grad_dl_tiles, dim3(static_cast<uint32_t>(n_vt * n_tblocks)),
                         dim3(kThreads), 0, stream, da);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    GemmArgs ga{};
    int nblk = 0;
    if (want_h) {
      // grad_hidden[N, H] (+)= D_c[N, width] . W_c[width, H]: P = W_c read
      // K-major (vocabulary rows), Q = D_c rows
      GemmOp& o = ga.op[ga.n_ops++];
      o.p = weight + static_cast<int64_t>(vocab0) * ldw;
      o.ldp = ldw;
      o.P = H;
      o.kext_p = v_rows;
      o.q = d;
      o.q_lo = d_lo;
      o.ldq = chunk;
      o.Q = static_cast<int>(N);
      o.kext_q = 0;
      o.K = width;
      o.q_kmajor = 0;
      o.out = grad_hidden;
      o.ldo = ld_gh;
      o.accumulate = c > 0;
      o.n_ptiles = n_htiles;
      o.n_qtiles = n_tblocks;
      o.first = nblk;
      nblk += static_cast<int>(round_up(static_cast<int64_t>(o.n_ptiles) * o.n_qtiles, 8));
    }
    if (want_w) {
      // grad_weight[vocab rows, H] = D_c^T . h: P = hidden and Q = D_c, both
      // read K-major (token rows)
      GemmOp& o = ga.op[ga.n_ops++];
      o.p = hw;
      o.ldp = ldhw;
      o.P = H;
      o.kext_p = static_cast<int>(N);
      o.q = d;
      o.q_lo = d_lo;
      o.ldq = chunk;
      o.Q = v_rows;
      o.kext_q = static_cast<int>(N);
      o.K = static_cast<int>(N);
      o.q_kmajor = 1;
      o.out = grad_weight + static_cast<int64_t>(vocab0) * ld_gw;
      o.ldo = ld_gw;
      o.accumulate = 0;
      o.n_ptiles = n_htiles;
      o.n_qtiles = (v_rows + kBQ - 1) / kBQ;
      o.first = nblk;
      nblk += o.n_ptiles * o.n_qtiles;
    }
    hipLaunchKernelGGL(grad_gemm_tiles, dim3(static_cast<uint32_t>(nblk)), dim3(kThreads), 0,
                       stream, ga);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rlk
