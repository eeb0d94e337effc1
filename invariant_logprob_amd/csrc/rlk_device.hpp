// Device-side building blocks shared by the logprob kernels (gfx950).
//
// Log-sum-exp state.  A partial reduction over a set of logits is kept as a
// pair (M, s) in base-2 units:
//     M = a rounded upper estimate of max(x) * log2(e)   (or -inf if empty)
//     s = sum_j 2^(x_j * log2(e) - M)                    (fp32)
// so that log(sum_j exp(x_j)) = ln(2) * (M + log2(s)).  Each term's exponent
// is formed by one fused multiply-add, x * log2(e) - M, rounded once, and M is
// the very value used as the offset, so its own rounding cancels out of the
// result.  Two pairs merge by rescaling to the larger M; the merge below is
// symmetric in its operands bit for bit (products formed separately, no
// contraction), so a butterfly leaves every lane with identical bits.
//
// Non-finite logits: -inf entries contribute 0 as long as one entry is
// finite; +inf or NaN anywhere makes the result NaN; an all -inf row gives
// NaN (log of 0 sum is -inf, and -inf - -inf is NaN in logp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// No implicit multiply-add contraction anywhere in the kernels: whether the
// compiler fuses a product into a neighbouring add would otherwise depend on
// how the surrounding code is laid out, and two kernels computing the same
// quantity could round it differently.  Fused multiply-adds are written out
// explicitly (__builtin_fmaf) where they are wanted.
#pragma clang fp contract(off)

namespace rlk {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// NaN-propagating maximum (IEEE 754-2019 maximum; v_maximum3_f32 on gfx950).
// Unlike fmaxf it needs no quieting of its inputs first, which fmaxf costs
// one instruction per value; a NaN logit still makes its row's result NaN
// (through its own exponential term as well).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load / store (data touched once: non-temporal hint)
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store16_stream(void* p, float a, float b, float c, float d) {
  f32x4_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 pair packed in a 32-bit word -> two exact fp32 values
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Offset used for the exponent of each term: an empty (-inf) state uses 0,
// so that -inf logits give 2^-inf = 0 instead of NaN.
__device__ __forceinline__ float lse_offset(float M) { return M == neg_inf() ? 0.0f : M; }

// Symmetric merge of (M, s) with (M2, s2).
__device__ __forceinline__ void lse_merge(float& M, float& s, float M2, float s2) {
#pragma clang fp contract(off)
  const float Mn = fmaxf(M, M2);
  const float a = (M == Mn) ? 1.0f : fast_exp2(M - Mn);
  const float b = (M2 == Mn) ? 1.0f : fast_exp2(M2 - Mn);
  const float p = s * a;
  const float q = s2 * b;
  s = p + q;
  M = Mn;
}

// Raise the offset of state (M, s) to cover a new block maximum given in
// natural units; returns the offset to use for the block's terms.
__device__ __forceinline__ float lse_raise(float& M, float& s, float block_max) {
  const float Mb = block_max * kLog2e;
  if (Mb > M) {
    s = (M == neg_inf()) ? s : s * fast_exp2(M - Mb);
    M = Mb;
  }
  return lse_offset(M);
}

// Term of the sum for logit x at offset Mu.
__device__ __forceinline__ float lse_term(float x, float Mu) {
  return fast_exp2(__builtin_fmaf(x, kLog2e, -Mu));
}

// Entropy-carrying state: t = sum_j 2^(x_j log2 e - M) x_j rides along with
// s under the same offset, so sum_j p_j x_j = t / s.
__device__ __forceinline__ void lse3_merge(float& M, float& s, float& t, float M2, float s2, float t2) {
#pragma clang fp contract(off)
  const float Mn = fmaxf(M, M2);
  const float a = (M == Mn) ? 1.0f : fast_exp2(M - Mn);
  const float b = (M2 == Mn) ? 1.0f : fast_exp2(M2 - Mn);
  const float p = s * a;
  const float q = s2 * b;
  const float u = t * a;
  const float w = t2 * b;
  s = p + q;
  t = u + w;
  M = Mn;
}

__device__ __forceinline__ float lse3_raise(float& M, float& s, float& t, float block_max) {
  const float Mb = block_max * kLog2e;
  if (Mb > M) {
    if (M != neg_inf()) {
      const float f = fast_exp2(M - Mb);
      s = s * f;
      t = t * f;
    }
    M = Mb;
  }
  return lse_offset(M);
}

// Natural-log LSE of a finished state.
__device__ __forceinline__ float lse_finish(float M, float s) {
#pragma clang fp contract(off)
  const float l2 = M + fast_log2(s);
  return l2 * kLn2;
}

// The value lane (lane ^ m) holds, for the six exchanges of the wave
// reduction: m = 32 and 16 through the gfx950 half-swap instructions
// (v_permlane32_swap / v_permlane16_swap, then a select of the half that
// came from the partner), m = 8 within each 16-lane row (DPP row_ror:8), m = 7
// within each 8-lane half row (DPP row_half_mirror), m = 2 and 1 within each
// quad (DPP quad_perm).  No LDS traffic; all lanes take part.
template <int K>
__device__ __forceinline__ float wave_partner(float v, int lane) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (K == 0) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  } else if constexpr (K == 1) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else if constexpr (K == 2) {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(u, 0x128, 0xF, 0xF, false));
  } else if constexpr (K == 3) {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(u, 0x141, 0xF, 0xF, false));
  } else if constexpr (K == 4) {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(u, 0x4E, 0xF, 0xF, false));
  } else {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(u, 0xB1, 0xF, 0xF, false));
  }
}

// Wave64 butterfly over the lane exchanges above, in the fixed order
// xor 32, 16, 8, 7, 2, 1 (these six masks span all 64 lanes): every lane ends
// with the merge of all 64 lanes, and since the merge is symmetric bit for
// bit, with the same bits.
template <int K = 0>
__device__ __forceinline__ void wave_lse_allreduce(float& M, float& s, int lane) {
  if constexpr (K < 6) {
    const float M2 = wave_partner<K>(M, lane);
    const float s2 = wave_partner<K>(s, lane);
    lse_merge(M, s, M2, s2);
    wave_lse_allreduce<K + 1>(M, s, lane);
  }
}

template <int K = 0>
__device__ __forceinline__ void wave_lse3_allreduce(float& M, float& s, float& t, int lane) {
  if constexpr (K < 6) {
    const float M2 = wave_partner<K>(M, lane);
    const float s2 = wave_partner<K>(s, lane);
    const float t2 = wave_partner<K>(t, lane);
    lse3_merge(M, s, t, M2, s2, t2);
    wave_lse3_allreduce<K + 1>(M, s, t, lane);
  }
}

}  // namespace rlk
