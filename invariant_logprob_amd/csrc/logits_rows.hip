// Selected-token logprob from materialised bf16 logits, and its backward.
//
// Forward (one workgroup per row; more rows than one launch's grid limit
// take further launches from the host, with the same per-row schedule).  The
// row is streamed once from HBM in 16-byte vectors of 8 bf16; a row of at
// most four steps (V <= 32768) is requested whole before it is consumed.  Vector k of a
// row always goes to thread k % kRowThreads and is visited in ascending k, so
// every lane's partial (M, s) is a function of the row's values and of V
// alone.  Lanes merge in a fixed wave64 butterfly over register lane
// exchanges, waves merge in ascending wave order through LDS.
// Nothing depends on N, on the row's index or on other rows: the batch
// invariance of page "[RFC] Batch-Invariant RL Kernel Suite for
// Train-Inference Consistency" (relation I) holds by construction, and there
// are no atomics (page "[WS1 Test] #154 dtype pin + ...", section
// "Workstream 3 - #153", scope item 2).
//
// Backward (grid = rows x column blocks of 8192).  Elementwise:
//   d[i, j] = g_i * ([j == t_i] - exp(x_ij - lse_i)),
// evaluated as fma(-g_i, p_ij, [j == t_i] g_i) with p_ij = 2^(x_ij log2 e -
// lse_i log2 e).  No reduction, so each element depends on its row only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"

namespace rlk {

namespace {

constexpr uint32_t kNegInfPair = 0xff80ff80u;  // two bf16 -inf

struct Vec8 {
  float v[8];
};

__device__ __forceinline__ Vec8 decode(const uint4& w) {
  Vec8 r;
  r.v[0] = bf16_lo(w.x);
  r.v[1] = bf16_hi(w.x);
  r.v[2] = bf16_lo(w.y);
  r.v[3] = bf16_hi(w.y);
  r.v[4] = bf16_lo(w.z);
  r.v[5] = bf16_hi(w.z);
  r.v[6] = bf16_lo(w.w);
  r.v[7] = bf16_hi(w.w);
  return r;
}

// Maximum of a lane's block of 8 U values: two chains of three-input maxima
// (the maximum is exact, so the grouping does not change the result).
template <int U>
__device__ __forceinline__ float block_max(const Vec8 (&x)[U]) {
  float m0 = vmax(vmax(x[0].v[0], x[0].v[1]), x[0].v[2]);
  float m1 = vmax(vmax(x[0].v[3], x[0].v[4]), x[0].v[5]);
  m0 = vmax(vmax(m0, x[0].v[6]), x[0].v[7]);
#pragma unroll
  for (int u = 1; u < U; ++u) {
    m1 = vmax(vmax(m1, x[u].v[0]), x[u].v[1]);
    m0 = vmax(vmax(m0, x[u].v[2]), x[u].v[3]);
    m1 = vmax(vmax(m1, x[u].v[4]), x[u].v[5]);
    m0 = vmax(vmax(m0, x[u].v[6]), x[u].v[7]);
  }
  return vmax(m0, m1);
}

// Sum of the 8 terms in a fixed pairwise tree.
__device__ __forceinline__ float sum8_terms(const Vec8& a, float Mu) {
#pragma clang fp contract(off)
  const float e0 = lse_term(a.v[0], Mu), e1 = lse_term(a.v[1], Mu);
  const float e2 = lse_term(a.v[2], Mu), e3 = lse_term(a.v[3], Mu);
  const float e4 = lse_term(a.v[4], Mu), e5 = lse_term(a.v[5], Mu);
  const float e6 = lse_term(a.v[6], Mu), e7 = lse_term(a.v[7], Mu);
  return ((e0 + e1) + (e2 + e3)) + ((e4 + e5) + (e6 + e7));
}

// One block of kUnroll vectors held by a lane: raise the offset to the
// block maximum, then add the block's terms in ascending vector order.
template <int U>
__device__ __forceinline__ void consume(float& M, float& s, const Vec8 (&x)[U]) {
#pragma clang fp contract(off)
  const float Mu = lse_raise(M, s, block_max<U>(x));
#pragma unroll
  for (int u = 0; u < U; ++u) s = s + sum8_terms(x[u], Mu);
}

// Entropy variant of consume: the same terms also weight the logits.  A -inf
// logit is clamped to -FLT_MAX for the product, so its zero term adds 0
// instead of 0 * -inf; the clamp is the NaN-propagating maximum (one
// instruction, no quieting of its input), and a NaN logit makes the row NaN
// through its own term either way.
__device__ __forceinline__ float sum8_weighted(const Vec8& a, float Mu, float& tsum) {
  float e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = lse_term(a.v[k], Mu);
  // weighted terms as one explicit multiply-add chain in element order
  float tw = e[0] * vmax(a.v[0], -3.402823466e38f);
#pragma unroll
  for (int k = 1; k < 8; ++k) tw = __builtin_fmaf(e[k], vmax(a.v[k], -3.402823466e38f), tw);
  tsum = tw;
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

template <int U>
__device__ __forceinline__ void consume3(float& M, float& s, float& t, const Vec8 (&x)[U]) {
#pragma clang fp contract(off)
  const float Mu = lse3_raise(M, s, t, block_max<U>(x));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float tw;
    const float se = sum8_weighted(x[u], Mu, tw);
    s = s + se;
    t = t + tw;
  }
}

template <int THREADS, int UNROLL, bool kEntropy, int kShort = 0>
__global__ __launch_bounds__(THREADS) void logp_fwd_rows(
    const uint16_t* __restrict__ logits, int64_t ld, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, int64_t row0, int V, float* __restrict__ logp,
    float* __restrict__ lse, float* __restrict__ ent) {
  constexpr int kWaves = THREADS / 64;
  const int64_t row = row0 + blockIdx.x;
  const int tid = threadIdx.x;
  if (mask != nullptr && mask[row] == 0) {
    if (tid == 0) {
      logp[row] = 0.0f;
      if (lse != nullptr) lse[row] = 0.0f;
      if constexpr (kEntropy) ent[row] = 0.0f;
    }
    return;
  }
  const uint16_t* rowp = logits + row * ld;
  const uint4* vp = reinterpret_cast<const uint4*>(rowp);
  // the target and its logit are loaded first, so that their latency hides
  // behind the row's stream instead of adding to the row's end
  int64_t t = -1;
  float xt = 0.0f;
  if (tid == 0) {
    t = targets[row];
    if (t >= 0 && t < V) xt = bf16_to_f32(rowp[t]);
  }
  const int nfull = V >> 3;                 // vectors lying wholly inside [0, V)
  const int nvec = (V + 7) >> 3;
  constexpr int kStep = THREADS * UNROLL;
  const int nmain = (nfull / kStep) * kStep;  // unguarded part

  float M = neg_inf();
  float s = 0.0f;
  float tw = 0.0f;  // entropy variant only
  if constexpr (kShort > 0) {
    // Short rows (at most kShort steps): every load of the row is issued
    // before the first is consumed, so the row costs one memory round trip
    // rather than one per step; the steps are then consumed in the same
    // order, with the same tail handling, as the loop below (the same bits).
    uint4 wv[kShort][UNROLL];
#pragma unroll
    for (int st = 0; st < kShort; ++st)
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = st * kStep + u * THREADS + tid;
        wv[st][u] = make_uint4(kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair);
        if (k < nvec) wv[st][u] = load16_stream(vp + k);
      }
#pragma unroll
    for (int st = 0; st < kShort; ++st) {
      const int base = st * kStep;
      if (base >= nvec) break;
      Vec8 x[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        x[u] = decode(wv[st][u]);
        const int k = base + u * THREADS + tid;
        if (base >= nmain && k == nfull) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (8 * k + e >= V) x[u].v[e] = neg_inf();
        }
      }
      if constexpr (kEntropy) consume3<UNROLL>(M, s, tw, x);
      else consume<UNROLL>(M, s, x);
    }
  } else {
  for (int base = 0; base < nmain; base += kStep) {
    uint4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) w[u] = load16_stream(vp + base + u * THREADS + tid);
    Vec8 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x[u] = decode(w[u]);
    if constexpr (kEntropy) consume3<UNROLL>(M, s, tw, x);
    else consume<UNROLL>(M, s, x);
  }
  if (nmain < nvec) {
    // guarded tail: same lane map (vector k -> thread k % THREADS)
    Vec8 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = nmain + u * THREADS + tid;
      uint4 w = make_uint4(kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair);
      if (k < nvec) w = vp[k];
      x[u] = decode(w);
      if (k == nfull) {  // the one vector straddling V (only when V % 8 != 0)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * k + e >= V) x[u].v[e] = neg_inf();
      }
    }
    if constexpr (kEntropy) consume3<UNROLL>(M, s, tw, x);
    else consume<UNROLL>(M, s, x);
  }
  }

  if constexpr (kEntropy) wave_lse3_allreduce(M, s, tw, tid & 63);
  else wave_lse_allreduce(M, s, tid & 63);
  __shared__ float sM[kWaves];
  __shared__ float sS[kWaves];
  __shared__ float sT[kWaves];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    sM[wave] = M;
    sS[wave] = s;
    if constexpr (kEntropy) sT[wave] = tw;
  }
  __syncthreads();
  if (tid == 0) {
    float Mt = sM[0];
    float st = sS[0];
    float tt = kEntropy ? sT[0] : 0.0f;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      if constexpr (kEntropy) lse3_merge(Mt, st, tt, sM[w], sS[w], sT[w]);
      else lse_merge(Mt, st, sM[w], sS[w]);
    }
    const float l = lse_finish(Mt, st);
    if constexpr (kEntropy) {
#pragma clang fp contract(off)
      ent[row] = l - tt / st;
    }
    const float lp = (t >= 0 && t < V) ? xt - l : __builtin_nanf("");
    logp[row] = lp;
    if (lse != nullptr) lse[row] = l;
  }
}

// Column blocks of the elementwise kernels (backward, dense log-softmax).
// Block L of the N x nb blocks covers row L / nb, 4-column groups
// [(L mod nb) * THREADS * UNROLL, + THREADS * UNROLL): consecutive blocks
// walk a row contiguously.  Workgroup ids are regrouped so that the blocks
// each XCD runs form one contiguous range (workgroups are dispatched
// round-robin over the 8 XCDs), and a grid-stride loop keeps the grid
// within launch limits for any N; the grid is a multiple of 8, so every
// iteration of a workgroup stays on its XCD.  Pure scheduling: each output
// element depends on its own row only.
__device__ __forceinline__ int64_t xcd_block(int64_t w, int64_t total) {
  const int64_t t8 = (total / 8) * 8;
  return (w < t8) ? (w & 7) * (t8 / 8) + (w >> 3) : w;
}

// Backward: thread handles groups of 4 columns (an 8-byte bf16 load, a
// 16-byte fp32 store), so every load and store instruction of a wave covers
// one contiguous span (512 B read, 1 KB written).
template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void logp_bwd_rows(
    const uint16_t* __restrict__ logits, int64_t ld, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, const float* __restrict__ lse,
    const float* __restrict__ grad, int64_t N, int V, int nb, float* __restrict__ dl,
    int64_t ldg) {
  const int tid = threadIdx.x;
  const int nq = (V + 3) >> 2;                  // 4-column groups
  const int64_t total = N * nb;
  const float nan = __builtin_nanf("");
  for (int64_t wid = blockIdx.x; wid < total; wid += gridDim.x) {
    const int64_t L = xcd_block(wid, total);
    const int64_t row = L / nb;
    const int qbase = static_cast<int>(L - row * nb) * (THREADS * UNROLL);
    float* outp = dl + row * ldg;
    const bool active = (mask == nullptr) || (mask[row] != 0);
    if (!active) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int q = qbase + u * THREADS + tid;
        if (q >= nq) break;
        const int j = 4 * q;
        if (j + 4 <= V) {
          store16_stream(outp + j, 0.f, 0.f, 0.f, 0.f);
        } else {
          for (int e = 0; j + e < V; ++e) outp[j + e] = 0.0f;
        }
      }
      continue;
    }
    const int64_t t = targets[row];
    const bool tvalid = (t >= 0 && t < V);
    const float g = grad[row];
    const float off = lse[row] * kLog2e;
    const float ng = -g;
    const uint2* vp = reinterpret_cast<const uint2*>(logits + row * ld);
    uint2 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      w[u] = make_uint2(kNegInfPair, kNegInfPair);
      if (q < nq) w[u] = load8_stream(vp + q);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      if (q >= nq) break;
      const int j = 4 * q;
      const float x[4] = {bf16_lo(w[u].x), bf16_hi(w[u].x), bf16_lo(w[u].y), bf16_hi(w[u].y)};
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = ng * fast_exp2(__builtin_fmaf(x[e], kLog2e, -off));
      if (t >= j && t < j + 4) {
        const int et = static_cast<int>(t - j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e == et) d[e] = __builtin_fmaf(ng, fast_exp2(__builtin_fmaf(x[e], kLog2e, -off)), g);
      }
      if (!tvalid) {
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = nan;
      }
      if (j + 4 <= V) {
        store16_stream(outp + j, d[0], d[1], d[2], d[3]);
      } else {
        for (int e = 0; j + e < V; ++e) outp[j + e] = d[e];
      }
    }
  }
}

// The backward from fp32 logits (the storing fused forward's output), with
// the access pattern and block order of logp_bwd_rows and the per-element
// arithmetic of the fused backward's epilogue:
//   d = fma(-g, 2^(fma(x, log2 e, -lse log2 e)), [j == t] g + poison)
// so that for the same logits and lse its output is bit-identical to the
// fused backward's.  A lane reads all of its elements before it writes any,
// and lanes own disjoint elements, so logits and dl may be one buffer.
template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void logp_bwd_rows_f32(
    const float* logits, int64_t ld, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, const float* __restrict__ lse,
    const float* __restrict__ grad, int64_t N, int V, int nb, float* dl, int64_t ldg) {
  const int tid = threadIdx.x;
  const int nq = (V + 3) >> 2;                  // 4-column groups
  const int64_t total = N * nb;
  const float nan = __builtin_nanf("");
  for (int64_t wid = blockIdx.x; wid < total; wid += gridDim.x) {
    const int64_t L = xcd_block(wid, total);
    const int64_t row = L / nb;
    const int qbase = static_cast<int>(L - row * nb) * (THREADS * UNROLL);
    float* outp = dl + row * ldg;
    const bool active = (mask == nullptr) || (mask[row] != 0);
    if (!active) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int q = qbase + u * THREADS + tid;
        if (q >= nq) break;
        const int j = 4 * q;
        if (j + 4 <= V) {
          store16_stream(outp + j, 0.f, 0.f, 0.f, 0.f);
        } else {
          for (int e = 0; j + e < V; ++e) outp[j + e] = 0.0f;
        }
      }
      continue;
    }
    const int64_t t = targets[row];
    const float g = grad[row];
    const float off = lse[row] * kLog2e;
    const float poison = (t >= 0 && t < V) ? 0.0f : nan;
    const float4* vp = reinterpret_cast<const float4*>(logits + row * ld);
    float4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      w[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < nq) w[u] = vp[q];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      if (q >= nq) break;
      const int j = 4 * q;
      const float x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(__builtin_fmaf(x[e], kLog2e, -off));
        const float add = (j + e == t) ? g : 0.0f;
        d[e] = __builtin_fmaf(-g, p, add + poison);
      }
      if (j + 4 <= V) {
        store16_stream(outp + j, d[0], d[1], d[2], d[3]);
      } else {
        for (int e = 0; j + e < V; ++e) outp[j + e] = d[e];
      }
    }
  }
}

// Dense log-softmax rows out[i, j] = x_ij - lse_i, with the backward's
// access pattern and block order.
template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void log_softmax_rows(
    const uint16_t* __restrict__ logits, int64_t ld, const uint8_t* __restrict__ mask,
    const float* __restrict__ lse, int64_t N, int V, int nb, float* __restrict__ out,
    int64_t ldo) {
  const int tid = threadIdx.x;
  const int nq = (V + 3) >> 2;
  const int64_t total = N * nb;
  for (int64_t wid = blockIdx.x; wid < total; wid += gridDim.x) {
    const int64_t L = xcd_block(wid, total);
    const int64_t row = L / nb;
    const int qbase = static_cast<int>(L - row * nb) * (THREADS * UNROLL);
    float* outp = out + row * ldo;
    const bool active = (mask == nullptr) || (mask[row] != 0);
    const float l = active ? lse[row] : 0.0f;
    const uint2* vp = reinterpret_cast<const uint2*>(logits + row * ld);
    uint2 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      w[u] = make_uint2(0u, 0u);
      if (active && q < nq) w[u] = load8_stream(vp + q);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int q = qbase + u * THREADS + tid;
      if (q >= nq) break;
      const int j = 4 * q;
      float d[4] = {bf16_lo(w[u].x) - l, bf16_hi(w[u].x) - l, bf16_lo(w[u].y) - l,
                    bf16_hi(w[u].y) - l};
      if (!active) d[0] = d[1] = d[2] = d[3] = 0.0f;
      if (j + 4 <= V) {
        store16_stream(outp + j, d[0], d[1], d[2], d[3]);
      } else {
        for (int e = 0; j + e < V; ++e) outp[j + e] = d[e];
      }
    }
  }
}

}  // namespace

// Compile-time schedule of the logits path.  These constants fix every row's
// reduction order; they are part of the build identity.
constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;
constexpr int kBwdThreads = 128;
constexpr int kBwdUnroll = 4;
// Upper bound on the elementwise kernels' grid (a multiple of 8); larger
// problems loop.
constexpr int64_t kBwdMaxGrid = int64_t(1) << 22;
// Rows per launch of the forward; more rows take further launches (the
// kernel stays a straight-line one-row program: no loop-carried state).
constexpr int64_t kRowMaxGrid = int64_t(1) << 22;
// Rows of at most this many steps (V <= 32768 at 256 threads x 4 vectors)
// have all their loads issued at once: a short row then costs one memory
// round trip instead of one per step.
constexpr int kShortSteps = 4;

int logits_schedule_threads() { return kRowThreads; }
int logits_schedule_unroll() { return kRowUnroll; }

hipError_t launch_logp_fwd_rows(const uint16_t* logits, int64_t ld, const int64_t* targets,
                                const uint8_t* mask, int64_t N, int V, float* logp, float* lse,
                                float* entropy, hipStream_t stream) {
  for (int64_t row0 = 0; row0 < N; row0 += kRowMaxGrid) {
    const uint32_t grid = static_cast<uint32_t>(N - row0 < kRowMaxGrid ? N - row0 : kRowMaxGrid);
    // rows of at most kShortSteps steps are requested whole (chosen by V)
    const bool short_rows = (V + 7) / 8 <= kShortSteps * kRowThreads * kRowUnroll;
    if (short_rows && entropy == nullptr) {
      hipLaunchKernelGGL((logp_fwd_rows<kRowThreads, kRowUnroll, false, kShortSteps>), dim3(grid),
                         dim3(kRowThreads), 0, stream, logits, ld, targets, mask, row0, V, logp,
                         lse, nullptr);
    } else if (short_rows) {
      hipLaunchKernelGGL((logp_fwd_rows<kRowThreads, kRowUnroll, true, kShortSteps>), dim3(grid),
                         dim3(kRowThreads), 0, stream, logits, ld, targets, mask, row0, V, logp,
                         lse, entropy);
    } else if (entropy == nullptr) {
      hipLaunchKernelGGL((logp_fwd_rows<kRowThreads, kRowUnroll, false>), dim3(grid),
                         dim3(kRowThreads), 0, stream, logits, ld, targets, mask, row0, V, logp,
                         lse, nullptr);
    } else {
      hipLaunchKernelGGL((logp_fwd_rows<kRowThreads, kRowUnroll, true>), dim3(grid),
                         dim3(kRowThreads), 0, stream, logits, ld, targets, mask, row0, V, logp,
                         lse, entropy);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static uint32_t elementwise_grid(int64_t total) {
  return static_cast<uint32_t>(total < kBwdMaxGrid ? total : kBwdMaxGrid);
}

hipError_t launch_logp_bwd_rows(const uint16_t* logits, int64_t ld, const int64_t* targets,
                                const uint8_t* mask, const float* lse, const float* grad, int64_t N,
                                int V, float* dl, int64_t ldg, hipStream_t stream) {
  const int nq = (V + 3) / 4;
  const int per_block = kBwdThreads * kBwdUnroll;
  const int nb = (nq + per_block - 1) / per_block;
  hipLaunchKernelGGL((logp_bwd_rows<kBwdThreads, kBwdUnroll>), dim3(elementwise_grid(N * nb)),
                     dim3(kBwdThreads), 0, stream, logits, ld, targets, mask, lse, grad, N, V, nb,
                     dl, ldg);
  return hipGetLastError();
}

hipError_t launch_logp_bwd_rows_f32(const float* logits, int64_t ld, const int64_t* targets,
                                    const uint8_t* mask, const float* lse, const float* grad,
                                    int64_t N, int V, float* dl, int64_t ldg, hipStream_t stream) {
  const int nq = (V + 3) / 4;
  const int per_block = kBwdThreads * kBwdUnroll;
  const int nb = (nq + per_block - 1) / per_block;
  hipLaunchKernelGGL((logp_bwd_rows_f32<kBwdThreads, kBwdUnroll>), dim3(elementwise_grid(N * nb)),
                     dim3(kBwdThreads), 0, stream, logits, ld, targets, mask, lse, grad, N, V, nb,
                     dl, ldg);
  return hipGetLastError();
}

hipError_t launch_log_softmax_rows(const uint16_t* logits, int64_t ld, const uint8_t* mask,
                                   const float* lse, int64_t N, int V, float* out, int64_t ldo,
                                   hipStream_t stream) {
  const int nq = (V + 3) / 4;
  const int per_block = kBwdThreads * kBwdUnroll;
  const int nb = (nq + per_block - 1) / per_block;
  hipLaunchKernelGGL((log_softmax_rows<kBwdThreads, kBwdUnroll>), dim3(elementwise_grid(N * nb)),
                     dim3(kBwdThreads), 0, stream, logits, ld, mask, lse, N, V, nb, out, ldo);
  return hipGetLastError();
}

}  // namespace rlk
