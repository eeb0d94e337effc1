// C ABI of the batch-invariant selected-token logprob library (include/rlk.h).
//
// Host side only: argument validation, then launches on the caller's
// stream.  How a row is reduced -- the kernel's arithmetic, its reduction
// schedule and order -- is chosen from V (and H) only, never from N, so the
// batch shape cannot change a row's bits (page "[RFC] Batch-Invariant RL
// Kernel Suite for Train-Inference Consistency", section "Problem": dispatch
// by shape is one of the named drift sources).  The one choice N makes is the
// fused kernels' launch form for batches of at most 128 rows, which runs the
// full tile's instruction sequence for those rows and yields the same bits.
// No allocation, no synchronisation, no mutable state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk.h"
#include "rlk_internal.hpp"


#ifndef RLK_GIT_REV
#define RLK_GIT_REV "unknown"
#endif

namespace {

constexpr int64_t kMaxV = int64_t(1) << 28;
constexpr int64_t kMaxH = int64_t(1) << 22;
constexpr int64_t kMaxN = (int64_t(1) << 31) - 1;
// The fused tiles address a 256-row slab of W or hidden with 32-bit byte
// offsets, which bounds the leading dimensions.
constexpr int64_t kMaxLinearLd = int64_t(1) << 22;
// A launch covers fewer than 2^32 work-items: one tile kernel launch (one
// workgroup of 512 threads per tile) holds fewer than 2^23 tiles.  The row
// kernels loop over rows beyond their grid and have no such bound.
constexpr int64_t kMaxTileGrid = int64_t(1) << 23;
constexpr int64_t kTile = rlk::kLinearVocabTile;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? RLK_OK : RLK_ERR_LAUNCH; }

int check_logits(const void* logits, int64_t ld, int64_t N, int64_t V) {
  if (logits == nullptr) return RLK_ERR_INVALID_ARG;
  if (ld < V) return RLK_ERR_INVALID_ARG;
  if ((ld % 8) != 0 || !aligned16(logits)) return RLK_ERR_UNSUPPORTED;
  if (N > 0 && ld > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}

int check_linear(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w, int64_t N,
                 int64_t V, int64_t H) {
  if (hidden == nullptr || weight == nullptr) return RLK_ERR_INVALID_ARG;
  if (H < 1) return RLK_ERR_INVALID_ARG;
  if (ld_h < H || ld_w < H) return RLK_ERR_INVALID_ARG;
  if (H > kMaxH || ld_h >= kMaxLinearLd || ld_w >= kMaxLinearLd) return RLK_ERR_UNSUPPORTED;
  if ((H % 8) != 0 || (ld_h % 8) != 0 || (ld_w % 8) != 0) return RLK_ERR_UNSUPPORTED;
  if (!aligned16(hidden) || !aligned16(weight)) return RLK_ERR_UNSUPPORTED;
  const int64_t tiles = ceil_div(V, rlk::kLinearVocabTile) * ceil_div(N, rlk::kLinearTokenTile);
  if (tiles >= kMaxTileGrid) return RLK_ERR_UNSUPPORTED;
  if (N > 0 && ld_h > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  if (ld_w > (int64_t(1) << 62) / V) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}

// An fp32 [N, ld] matrix (rows of ld elements, V of them used).
int check_f32_rows(const void* p, int64_t ld, int64_t N, int64_t V) {
  if (p == nullptr) return RLK_ERR_INVALID_ARG;
  if (ld < V) return RLK_ERR_INVALID_ARG;
  if ((ld % 4) != 0 || !aligned16(p)) return RLK_ERR_UNSUPPORTED;
  if (N > 0 && ld > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}

// Whether the byte spans of two row-major [N, ld] matrices (V elements of
// each row used, N >= 1) intersect.
bool rows_overlap(const void* a, int64_t lda, size_t asz, const void* b, int64_t ldb, size_t bsz,
                  int64_t N, int64_t V) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
  const uintptr_t a1 = a0 + static_cast<uintptr_t>((N - 1) * lda + V) * asz;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t b1 = b0 + static_cast<uintptr_t>((N - 1) * ldb + V) * bsz;
  return a0 < b1 && b0 < a1;
}

int check_sizes(int64_t N, int64_t V) {
  if (N < 0 || V < 1) return RLK_ERR_INVALID_ARG;
  if (N > kMaxN || V > kMaxV) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}


// Both parameter-gradient entry points: logits null (recomputed per chunk)
// or the fp32 logits the forward kept.
int param_grads(const float* logits, int64_t ld_z, const void* hidden, int64_t ld_h,
                const void* weight, int64_t ld_w, const int64_t* targets, const uint8_t* mask,
                const float* lse, const float* grad_logp, int64_t N, int64_t V, int64_t H,
                float* grad_hidden, int64_t ld_gh, float* grad_weight, int64_t ld_gw,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (grad_hidden == nullptr && grad_weight == nullptr) return RLK_ERR_INVALID_ARG;
  if (weight == nullptr || H < 1 || ld_w < H) return RLK_ERR_INVALID_ARG;
  if (grad_weight != nullptr) {
    if (ld_gw < H) return RLK_ERR_INVALID_ARG;
    if ((ld_gw % 4) != 0 || !aligned16(grad_weight)) return RLK_ERR_UNSUPPORTED;
    if (ld_gw > (int64_t(1) << 62) / V) return RLK_ERR_UNSUPPORTED;
  }
  if (N == 0) {
    if ((H % 8) != 0) return RLK_ERR_UNSUPPORTED;
    return status_of(rlk::launch_linear_param_grads(
        nullptr, 0, static_cast<const uint16_t*>(weight), ld_w, nullptr, nullptr, nullptr, nullptr,
        0, static_cast<int>(V), static_cast<int>(H), nullptr, 0, grad_weight, ld_gw, nullptr, 0,
        nullptr, stream));
  }
  if (targets == nullptr || lse == nullptr || grad_logp == nullptr || workspace == nullptr)
    return RLK_ERR_INVALID_ARG;
  st = check_linear(hidden, ld_h, weight, ld_w, N, V, H);
  if (st != RLK_OK) return st;
  // the transposed hidden's rows (N rounded up to 8) are addressed like a
  // fused-tile operand
  if (N > kMaxLinearLd - 16) return RLK_ERR_UNSUPPORTED;
  {
    // the largest launch of the path: one chunk's two products, grad_hidden
    // tiles (rounded up to 8) then grad_weight tiles
    const int64_t htiles = ceil_div(H, kTile);
    const int64_t chunk_tiles = ceil_div(V < rlk::kGradChunk ? V : rlk::kGradChunk, kTile);
    const int64_t grid = ceil_div(htiles * ceil_div(N, kTile), 8) * 8 + htiles * chunk_tiles;
    if (grid >= kMaxTileGrid) return RLK_ERR_UNSUPPORTED;
  }
  if (grad_hidden != nullptr) {
    if (ld_gh < H) return RLK_ERR_INVALID_ARG;
    if ((ld_gh % 4) != 0 || !aligned16(grad_hidden)) return RLK_ERR_UNSUPPORTED;
    if (ld_gh > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  }
  if (logits != nullptr) {
    st = check_f32_rows(logits, ld_z, N, V);
    if (st != RLK_OK) return st;
  }
  if (workspace_bytes < rlk::linear_param_grads_workspace_bytes(N, V, H)) return RLK_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return RLK_ERR_UNSUPPORTED;
  return status_of(rlk::launch_linear_param_grads(
      static_cast<const uint16_t*>(hidden), ld_h, static_cast<const uint16_t*>(weight), ld_w,
      targets, mask, lse, grad_logp, N, static_cast<int>(V), static_cast<int>(H), grad_hidden,
      ld_gh, grad_weight, ld_gw, logits, ld_z, workspace, stream));
}

}  // namespace

namespace rlk {

// Validation shared by rlk_linear_logp and its allocation-free variant
// (everything but the workspace).
int check_linear_logp_args(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                           const int64_t* targets, const float* logp, int64_t N, int64_t V,
                           int64_t H) {
  const int st = check_sizes(N, V);
  if (st != RLK_OK || N == 0) return st;
  if (targets == nullptr || logp == nullptr) return RLK_ERR_INVALID_ARG;
  return check_linear(hidden, ld_h, weight, ld_w, N, V, H);
}

}  // namespace rlk

extern "C" {

int rlk_logp_selected(const void* logits, int64_t ld, const int64_t* targets, const uint8_t* mask,
                      int64_t N, int64_t V, float* logp, float* lse, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (targets == nullptr || logp == nullptr) return RLK_ERR_INVALID_ARG;
  st = check_logits(logits, ld, N, V);
  if (st != RLK_OK) return st;
  return status_of(rlk::launch_logp_fwd_rows(static_cast<const uint16_t*>(logits), ld, targets,
                                             mask, N, static_cast<int>(V), logp, lse, nullptr,
                                             stream));
}

int rlk_logp_entropy(const void* logits, int64_t ld, const int64_t* targets, const uint8_t* mask,
                     int64_t N, int64_t V, float* logp, float* lse, float* entropy,
                     hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (targets == nullptr || logp == nullptr || entropy == nullptr) return RLK_ERR_INVALID_ARG;
  st = check_logits(logits, ld, N, V);
  if (st != RLK_OK) return st;
  return status_of(rlk::launch_logp_fwd_rows(static_cast<const uint16_t*>(logits), ld, targets,
                                             mask, N, static_cast<int>(V), logp, lse, entropy,
                                             stream));
}

int rlk_log_softmax(const void* logits, int64_t ld, const uint8_t* mask, const float* lse,
                    int64_t N, int64_t V, float* out, int64_t ld_out, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (lse == nullptr || out == nullptr) return RLK_ERR_INVALID_ARG;
  if (ld_out < V) return RLK_ERR_INVALID_ARG;
  if ((ld_out % 4) != 0 || !aligned16(out)) return RLK_ERR_UNSUPPORTED;
  if (ld_out > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  st = check_logits(logits, ld, N, V);
  if (st != RLK_OK) return st;
  if (rows_overlap(logits, ld, 2, out, ld_out, sizeof(float), N, V)) return RLK_ERR_INVALID_ARG;
  return status_of(rlk::launch_log_softmax_rows(static_cast<const uint16_t*>(logits), ld, mask, lse,
                                                N, static_cast<int>(V), out, ld_out, stream));
}

size_t rlk_linear_logp_workspace_size(int64_t N, int64_t V, int64_t H) {
  (void)H;
  if (N < 0 || V < 1) return 0;
  return rlk::linear_workspace_bytes(N, V);
}

int rlk_linear_logp(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                    const int64_t* targets, const uint8_t* mask, int64_t N, int64_t V, int64_t H,
                    float* logp, float* lse, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  const int st = rlk::check_linear_logp_args(hidden, ld_h, weight, ld_w, targets, logp, N, V, H);
  if (st != RLK_OK || N == 0) return st;
  if (workspace == nullptr) return RLK_ERR_INVALID_ARG;
  if (workspace_bytes < rlk::linear_workspace_bytes(N, V)) return RLK_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return RLK_ERR_UNSUPPORTED;
  return status_of(rlk::launch_linear_logp(
      static_cast<const uint16_t*>(hidden), ld_h, static_cast<const uint16_t*>(weight), ld_w,
      targets, mask, N, static_cast<int>(V), static_cast<int>(H), logp, lse, nullptr, 0,
      workspace, stream));
}

int rlk_linear_logp_with_logits(const void* hidden, int64_t ld_h, const void* weight,
                                int64_t ld_w, const int64_t* targets, const uint8_t* mask,
                                int64_t N, int64_t V, int64_t H, float* logp, float* lse,
                                float* logits, int64_t ld_z, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (targets == nullptr || logp == nullptr || workspace == nullptr) return RLK_ERR_INVALID_ARG;
  st = check_linear(hidden, ld_h, weight, ld_w, N, V, H);
  if (st != RLK_OK) return st;
  st = check_f32_rows(logits, ld_z, N, V);
  if (st != RLK_OK) return st;
  if (workspace_bytes < rlk::linear_workspace_bytes(N, V)) return RLK_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return RLK_ERR_UNSUPPORTED;
  return status_of(rlk::launch_linear_logp(
      static_cast<const uint16_t*>(hidden), ld_h, static_cast<const uint16_t*>(weight), ld_w,
      targets, mask, N, static_cast<int>(V), static_cast<int>(H), logp, lse, logits, ld_z,
      workspace, stream));
}

int rlk_logp_backward_f32(const float* logits, int64_t ld, const int64_t* targets,
                          const uint8_t* mask, const float* lse, const float* grad_logp, int64_t N,
                          int64_t V, float* grad_logits, int64_t ld_g, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (targets == nullptr || lse == nullptr || grad_logp == nullptr) return RLK_ERR_INVALID_ARG;
  st = check_f32_rows(logits, ld, N, V);
  if (st != RLK_OK) return st;
  st = check_f32_rows(grad_logits, ld_g, N, V);
  if (st != RLK_OK) return st;
  // In place (the same buffer and stride) or disjoint; any other overlap of
  // the two [N, ld] spans would let a lane overwrite another lane's input.
  if ((grad_logits != logits || ld_g != ld) &&
      rows_overlap(logits, ld, sizeof(float), grad_logits, ld_g, sizeof(float), N, V))
    return RLK_ERR_INVALID_ARG;
  return status_of(rlk::launch_logp_bwd_rows_f32(logits, ld, targets, mask, lse, grad_logp, N,
                                                 static_cast<int>(V), grad_logits, ld_g, stream));
}

int rlk_logp_backward(const void* logits, int64_t ld, const void* hidden, int64_t ld_h,
                      const void* weight, int64_t ld_w, int64_t H, const int64_t* targets,
                      const uint8_t* mask, const float* lse, const float* grad_logp, int64_t N,
                      int64_t V, float* grad_logits, int64_t ld_g, hipStream_t stream) {
  int st = check_sizes(N, V);
  if (st != RLK_OK) return st;
  if (N == 0) return RLK_OK;
  if (targets == nullptr || lse == nullptr || grad_logp == nullptr || grad_logits == nullptr)
    return RLK_ERR_INVALID_ARG;
  if (ld_g < V) return RLK_ERR_INVALID_ARG;
  if ((ld_g % 4) != 0 || !aligned16(grad_logits)) return RLK_ERR_UNSUPPORTED;
  if (ld_g > (int64_t(1) << 62) / N) return RLK_ERR_UNSUPPORTED;
  if (logits != nullptr) {
    st = check_logits(logits, ld, N, V);
    if (st != RLK_OK) return st;
    // bf16 in, fp32 out: no overlap can be safe
    if (rows_overlap(logits, ld, 2, grad_logits, ld_g, sizeof(float), N, V))
      return RLK_ERR_INVALID_ARG;
    return status_of(rlk::launch_logp_bwd_rows(static_cast<const uint16_t*>(logits), ld, targets,
                                               mask, lse, grad_logp, N, static_cast<int>(V),
                                               grad_logits, ld_g, stream));
  }
  st = check_linear(hidden, ld_h, weight, ld_w, N, V, H);
  if (st != RLK_OK) return st;
  return status_of(rlk::launch_linear_dlogits(
      static_cast<const uint16_t*>(hidden), ld_h, static_cast<const uint16_t*>(weight), ld_w,
      targets, mask, lse, grad_logp, N, static_cast<int>(V), static_cast<int>(H), grad_logits,
      ld_g, stream));
}

size_t rlk_linear_logp_param_grads_workspace_size(int64_t N, int64_t V, int64_t H) {
  if (N < 0 || V < 1 || H < 1) return 0;
  return rlk::linear_param_grads_workspace_bytes(N, V, H);
}

int rlk_linear_logp_param_grads(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                const int64_t* targets, const uint8_t* mask, const float* lse,
                                const float* grad_logp, int64_t N, int64_t V, int64_t H,
                                float* grad_hidden, int64_t ld_gh, float* grad_weight,
                                int64_t ld_gw, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return param_grads(nullptr, 0, hidden, ld_h, weight, ld_w, targets, mask, lse, grad_logp, N, V,
                     H, grad_hidden, ld_gh, grad_weight, ld_gw, workspace, workspace_bytes, stream);
}

int rlk_linear_logp_param_grads_from_logits(const float* logits, int64_t ld_z, const void* hidden,
                                            int64_t ld_h, const void* weight, int64_t ld_w,
                                            const int64_t* targets, const uint8_t* mask,
                                            const float* lse, const float* grad_logp, int64_t N,
                                            int64_t V, int64_t H, float* grad_hidden,
                                            int64_t ld_gh, float* grad_weight, int64_t ld_gw,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  if (logits == nullptr && N > 0) return RLK_ERR_INVALID_ARG;
  return param_grads(logits, ld_z, hidden, ld_h, weight, ld_w, targets, mask, lse, grad_logp, N, V,
                     H, grad_hidden, ld_gh, grad_weight, ld_gw, workspace, workspace_bytes, stream);
}

int rlk_token_losses(const float* logp, const float* logp_old, const float* logp_ref,
                     const float* advantages, const uint8_t* mask, int64_t N, float eps_lo,
                     float eps_hi, float beta, float* ratio, float* loss, float* kl,
                     float* grad_logp, hipStream_t stream) {
  if (N < 0) return RLK_ERR_INVALID_ARG;
  if (N > kMaxN) return RLK_ERR_UNSUPPORTED;
  if (N == 0) return RLK_OK;
  if (logp == nullptr || logp_old == nullptr || advantages == nullptr) return RLK_ERR_INVALID_ARG;
  if (ratio == nullptr && loss == nullptr && kl == nullptr && grad_logp == nullptr)
    return RLK_ERR_INVALID_ARG;
  if (!(eps_lo >= 0.0f && eps_lo < 1.0f) || !(eps_hi >= 0.0f) || !(beta >= 0.0f))
    return RLK_ERR_INVALID_ARG;
  rlk::TokenLossArgs a{logp, logp_old, logp_ref, advantages, mask, N, eps_lo, eps_hi, beta,
                       ratio, loss, kl, grad_logp};
  return status_of(rlk::launch_token_losses(a, stream));
}

// The gate report names its backend and any failure reason (page "[WS1
// Test] #154 dtype pin + #152 KV path + #153 bwd invariance + #150 chain
// gate", section "Workstream 4 - #150", gate report contents): a status code
// is turned into the name a report can carry.
const char* rlk_status_string(int status) {
  switch (status) {
    case RLK_OK: return "RLK_OK";
    case RLK_ERR_INVALID_ARG: return "RLK_ERR_INVALID_ARG";
    case RLK_ERR_UNSUPPORTED: return "RLK_ERR_UNSUPPORTED";
    case RLK_ERR_LAUNCH: return "RLK_ERR_LAUNCH";
    default: return "unknown";
  }
}

#define RLK_STR2(x) #x
#define RLK_STR(x) RLK_STR2(x)

// The actual backend a gate report records beside the requested one (same
// page and section as above).

const char* rlk_build_info(void) {
  return "rlk 0.1.0; arch=gfx950; rev=" RLK_GIT_REV
         "; schedule=rows:256thr,4x16B/lane-step,whole-row-if<=4steps,bfly:pl32,pl16,ror8,hmir,qp2,qp1; bwd:128thr,4x8B,xcd-ordered; tile:" RLK_STR(256) "x" RLK_STR(
             256) "x" RLK_STR(64) ",8waves,mfma32x32x16bf16,2stage,group8,wg-per-tile; fused-n<=128:2-8waves,reg-staged-w,1stage,2-4wg-per-cu; combine:wave-per-row; grads:chunk" RLK_STR(16384) ",dl-bf16x2,kmajor-tr16";
}

}  // extern "C"
