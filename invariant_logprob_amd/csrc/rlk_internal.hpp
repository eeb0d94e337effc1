// Internal launchers behind the C ABI (include/rlk.h) and the compile-time
// schedule constants that fix every reduction order.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rlk {

// Fused path tile schedule: 256 vocabulary entries x 256 tokens per tile,
// K in stages of 64.  The vocabulary tile is also the log-sum-exp chunk.
constexpr int kLinearVocabTile = 256;
constexpr int kLinearTokenTile = 256;
constexpr int kLinearKStage = 64;
// Vocabulary tiles grouped together in the launch order (scheduling only).
constexpr int kLinearVocabGroup = 8;
// Vocabulary entries per pass of the parameter-gradient path (a multiple of
// the vocabulary tile): the chunking of the contraction over the vocabulary.
constexpr int kGradChunk = 16384;

int logits_schedule_threads();
int logits_schedule_unroll();

hipError_t launch_logp_fwd_rows(const uint16_t* logits, int64_t ld, const int64_t* targets,
                                const uint8_t* mask, int64_t N, int V, float* logp, float* lse,
                                float* entropy, hipStream_t stream);

hipError_t launch_log_softmax_rows(const uint16_t* logits, int64_t ld, const uint8_t* mask,
                                   const float* lse, int64_t N, int V, float* out, int64_t ldo,
                                   hipStream_t stream);

hipError_t launch_logp_bwd_rows(const uint16_t* logits, int64_t ld, const int64_t* targets,
                                const uint8_t* mask, const float* lse, const float* grad, int64_t N,
                                int V, float* dl, int64_t ldg, hipStream_t stream);
// The same backward from fp32 logits (as the storing fused forward writes
// them), with the fused backward's arithmetic, so its output is bit-identical
// to launch_linear_dlogits' for the same logits.  logits and dl may be the
// same buffer (ld == ldg).
hipError_t launch_logp_bwd_rows_f32(const float* logits, int64_t ld, const int64_t* targets,
                                    const uint8_t* mask, const float* lse, const float* grad,
                                    int64_t N, int V, float* dl, int64_t ldg, hipStream_t stream);

size_t linear_workspace_bytes(int64_t N, int64_t V);

// Argument checks of the fused forward, all but its workspace: an rlk_status
// (RLK_OK for N == 0, which launches nothing).
int check_linear_logp_args(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                           const int64_t* targets, const float* logp, int64_t N, int64_t V,
                           int64_t H);

struct TokenLossArgs {
  const float* logp;
  const float* logp_old;
  const float* logp_ref;  // may be null: no KL term
  const float* adv;
  const uint8_t* mask;
  int64_t N;
  float eps_lo;
  float eps_hi;
  float beta;
  float* ratio;
  float* loss;
  float* kl;
  float* grad;
};

hipError_t launch_token_losses(const TokenLossArgs& a, hipStream_t stream);

// logits may be null; otherwise the forward also writes the fp32 logits
// [N, ldz] (every row below N, columns below V).
hipError_t launch_linear_logp(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                              int64_t ldw, const int64_t* targets, const uint8_t* mask, int64_t N,
                              int V, int H, float* logp, float* lse, float* logits, int64_t ldz,
                              void* workspace, hipStream_t stream);

hipError_t launch_linear_dlogits(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                                 int64_t ldw, const int64_t* targets, const uint8_t* mask,
                                 const float* lse, const float* grad, int64_t N, int V, int H,
                                 float* dl, int64_t ldg, hipStream_t stream);

size_t linear_param_grads_workspace_bytes(int64_t N, int64_t V, int64_t H);

// logits may be null (the logits are recomputed per chunk); otherwise they
// are the fp32 [N, ldz] logits the forward kept, and each chunk's D is
// formed from them.  The gradients are bit-identical either way.
hipError_t launch_linear_param_grads(const uint16_t* hidden, int64_t ldh, const uint16_t* weight,
                                     int64_t ldw, const int64_t* targets, const uint8_t* mask,
                                     const float* lse, const float* grad, int64_t N, int V, int H,
                                     float* grad_hidden, int64_t ld_gh, float* grad_weight,
                                     int64_t ld_gw, const float* logits, int64_t ldz,
                                     void* workspace, hipStream_t stream);

}  // namespace rlk
