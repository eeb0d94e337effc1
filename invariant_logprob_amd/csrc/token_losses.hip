// Per-token loss terms consuming the selected logprob (GRPO / PPO form).
//
// The pages put the loss reductions (grpo_loss, ratio_kl) at the end of the
// operator chain and ask that, for bitwise invariance, they be per-token
// outputs rather than batch-normalised reductions (page "docs(ws1):
// batch-invariance contract RFC", section "First-Divergence Localization",
// review of the chain's last entry).  Per token i:
//   ratio = exp(logp - logp_old)
//   surr  = -min(ratio A, clip(ratio, 1 - eps_lo, 1 + eps_hi) A)
//   kl    = exp(ref - logp) - (ref - logp) - 1        (k3 estimator)
//   loss  = surr + beta kl
//   grad  = d loss / d logp  (0 through the clipped branch when min() picks it)
// Elementwise: each token's outputs depend on its own inputs only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_device.hpp"
#include "rlk_internal.hpp"

namespace rlk {

namespace {

__global__ __launch_bounds__(256) void token_losses_kernel(TokenLossArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.N) return;
  const bool active = (a.mask == nullptr) || (a.mask[i] != 0);
  float ratio = 0.0f, loss = 0.0f, kl = 0.0f, grad = 0.0f;
  if (active) {
    const float lp = a.logp[i];
    const float adv = a.adv[i];
    ratio = expf(lp - a.logp_old[i]);
    const float c = fminf(fmaxf(ratio, 1.0f - a.eps_lo), 1.0f + a.eps_hi);
    const float u = ratio * adv;
    const float v = c * adv;
    loss = -fminf(u, v);
    grad = (u <= v) ? -(adv * ratio) : 0.0f;
    if (a.logp_ref != nullptr) {
      const float d = a.logp_ref[i] - lp;
      const float em1 = expm1f(d);
      kl = em1 - d;
      loss = loss + a.beta * kl;
      grad = grad - a.beta * em1;
    }
  }
  if (a.ratio != nullptr) a.ratio[i] = ratio;
  if (a.loss != nullptr) a.loss[i] = loss;
  if (a.kl != nullptr) a.kl[i] = kl;
  if (a.grad != nullptr) a.grad[i] = grad;
}

}  // namespace

hipError_t launch_token_losses(const TokenLossArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(token_losses_kernel, dim3(static_cast<uint32_t>((a.N + 255) / 256)), dim3(256),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
