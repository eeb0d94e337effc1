// Host-only check of the C ABI's argument validation under AddressSanitizer
// and UndefinedBehaviorSanitizer.  csrc/rlk_api.hip is compiled for the host
// alone and linked against the stand-in launchers below, which record that a
// launch was reached and touch no device.  Every entry point is called with
// fake, never dereferenced addresses: invalid arguments must return the
// documented status with no launch, valid ones must reach exactly one
// launcher, and sizes at the limits must not overflow the validation
// arithmetic (UBSan turns a signed overflow into a failure).
#include <stdint.h>
#include <stdio.h>

#include "rlk.h"
#include "rlk_internal.hpp"

namespace {
int g_launches = 0;
int64_t g_N = -1;
int g_V = -1;

hipError_t record(int64_t N, int V) {
  ++g_launches;
  g_N = N;
  g_V = V;
  return hipSuccess;
}
}  // namespace

namespace rlk {
int logits_schedule_threads() { return 256; }
int logits_schedule_unroll() { return 8; }
hipError_t launch_logp_fwd_rows(const uint16_t*, int64_t, const int64_t*, const uint8_t*,
                                int64_t N, int V, float*, float*, float*, hipStream_t) {
  return record(N, V);
}
hipError_t launch_log_softmax_rows(const uint16_t*, int64_t, const uint8_t*, const float*,
                                   int64_t N, int V, float*, int64_t, hipStream_t) {
  return record(N, V);
}
hipError_t launch_logp_bwd_rows(const uint16_t*, int64_t, const int64_t*, const uint8_t*,
                                const float*, const float*, int64_t N, int V, float*, int64_t,
                                hipStream_t) {
  return record(N, V);
}
hipError_t launch_logp_bwd_rows_f32(const float*, int64_t, const int64_t*, const uint8_t*,
                                    const float*, const float*, int64_t N, int V, float*, int64_t,
                                    hipStream_t) {
  return record(N, V);
}
size_t linear_workspace_bytes(int64_t N, int64_t V) {
  return static_cast<size_t>(N) * static_cast<size_t>((V + 255) / 256) * 8 + 256;
}
hipError_t launch_token_losses(const TokenLossArgs& a, hipStream_t) { return record(a.N, 0); }
hipError_t launch_linear_logp(const uint16_t*, int64_t, const uint16_t*, int64_t, const int64_t*,
                              const uint8_t*, int64_t N, int V, int, float*, float*, float*,
                              int64_t, void*, hipStream_t) {
  return record(N, V);
}
hipError_t launch_linear_dlogits(const uint16_t*, int64_t, const uint16_t*, int64_t,
                                 const int64_t*, const uint8_t*, const float*, const float*,
                                 int64_t N, int V, int, float*, int64_t, hipStream_t) {
  return record(N, V);
}
size_t linear_param_grads_workspace_bytes(int64_t N, int64_t, int64_t) {
  return static_cast<size_t>(N) * 16384 * 2;
}
hipError_t launch_linear_param_grads(const uint16_t*, int64_t, const uint16_t*, int64_t,
                                     const int64_t*, const uint8_t*, const float*, const float*,
                                     int64_t N, int V, int, float*, int64_t, float*, int64_t,
                                     const float*, int64_t, void*, hipStream_t) {
  return record(N, V);
}
}  // namespace rlk

namespace {
int fails = 0;

// status must equal want, and a launch must have happened exactly when
// want is RLK_OK and `launches` says so
void expect(int status, int want, bool launches, const char* what) {
  static int seen = 0;
  const bool launched = g_launches != seen;
  seen = g_launches;
  if (status != want || launched != launches) {
    printf("FAIL %s: status %d (want %d), launched %d (want %d)\n", what, status, want,
           static_cast<int>(launched), static_cast<int>(launches));
    ++fails;
  }
}

void* at(uintptr_t a) { return reinterpret_cast<void*>(a); }
}  // namespace

int main() {
  const uintptr_t A = 0x100000;  // 16-byte aligned fake device address
  const int64_t* t = static_cast<const int64_t*>(at(A));
  float* f = static_cast<float*>(at(A + 0x10000000));
  float* g = static_cast<float*>(at(A + 0x20000000));
  const void* x = at(A);
  const int64_t kMaxN = (int64_t(1) << 31) - 1;

  // logits forward
  expect(rlk_logp_selected(x, 1024, t, nullptr, 4, 1024, f, nullptr, nullptr), RLK_OK, true,
         "logp: valid");
  expect(rlk_logp_selected(x, 1024, t, nullptr, 0, 1024, f, nullptr, nullptr), RLK_OK, false,
         "logp: N = 0");
  expect(rlk_logp_selected(x, 1024, t, nullptr, -1, 1024, f, nullptr, nullptr),
         RLK_ERR_INVALID_ARG, false, "logp: N < 0");
  expect(rlk_logp_selected(x, 1028, t, nullptr, 4, 1024, f, nullptr, nullptr),
         RLK_ERR_UNSUPPORTED, false, "logp: ld % 8");
  expect(rlk_logp_selected(at(A + 2), 1024, t, nullptr, 4, 1024, f, nullptr, nullptr),
         RLK_ERR_UNSUPPORTED, false, "logp: misaligned");
  expect(rlk_logp_selected(x, int64_t(1) << 40, t, nullptr, kMaxN, 1024, f, nullptr, nullptr),
         RLK_ERR_UNSUPPORTED, false, "logp: N x ld beyond 2^62");
  expect(rlk_logp_selected(x, int64_t(1) << 28, t, nullptr, int64_t(1) << 20, int64_t(1) << 28, f,
                           nullptr, nullptr),
         RLK_OK, true, "logp: V = 2^28");
  expect(rlk_logp_selected(x, int64_t(1) << 62, t, nullptr, 3, 1024, f, nullptr, nullptr),
         RLK_ERR_UNSUPPORTED, false, "logp: ld near 2^62");
  expect(rlk_logp_selected(x, int64_t(1) << 62, t, nullptr, 1, 1024, f, nullptr, nullptr),
         RLK_OK, true, "logp: one row, ld = 2^62");
  expect(rlk_logp_selected(x, INT64_MAX - 7, t, nullptr, 1, 1024, f, nullptr, nullptr),
         RLK_ERR_UNSUPPORTED, false, "logp: one row, ld beyond 2^62");
  expect(rlk_logp_entropy(x, 1024, t, nullptr, 4, 1024, f, nullptr, g, nullptr), RLK_OK, true,
         "entropy: valid");
  // dense log-softmax: bf16 in, fp32 out, no overlap allowed
  expect(rlk_log_softmax(x, 1024, nullptr, f, 4, 1024, g, 1024, nullptr), RLK_OK, true,
         "log_softmax: valid");
  expect(rlk_log_softmax(x, 1024, nullptr, f, 4, 1024, static_cast<float*>(at(A + 16)), 1024,
                         nullptr),
         RLK_ERR_INVALID_ARG, false, "log_softmax: overlap");
  expect(rlk_log_softmax(x, 1024, nullptr, f, kMaxN, 1024, g, int64_t(1) << 40, nullptr),
         RLK_ERR_UNSUPPORTED, false, "log_softmax: N x ld_out beyond 2^62");

  // logits backward
  expect(rlk_logp_backward(x, 1024, nullptr, 0, nullptr, 0, 0, t, nullptr, f, f, 4, 1024, g, 1024,
                           nullptr),
         RLK_OK, true, "bwd: valid");
  expect(rlk_logp_backward(x, 1024, nullptr, 0, nullptr, 0, 0, t, nullptr, f, f, 4, 1024,
                           static_cast<float*>(at(A + 4096)), 1024, nullptr),
         RLK_ERR_INVALID_ARG, false, "bwd: output overlaps the logits");
  expect(rlk_logp_backward(x, 1024, nullptr, 0, nullptr, 0, 0, t, nullptr, nullptr, f, 4, 1024, g,
                           1024, nullptr),
         RLK_ERR_INVALID_ARG, false, "bwd: no lse");
  expect(rlk_logp_backward(x, 1024, nullptr, 0, nullptr, 0, 0, t, nullptr, f, f, 4, 1024, g, 1026,
                           nullptr),
         RLK_ERR_UNSUPPORTED, false, "bwd: ld_g % 4");
  // fp32 backward: in place allowed, partial overlap refused
  expect(rlk_logp_backward_f32(f, 1024, t, nullptr, g, g, 4, 1000, f, 1024, nullptr), RLK_OK, true,
         "bwd f32: in place");
  expect(rlk_logp_backward_f32(f, 1024, t, nullptr, g, g, 4, 1000, f + 16, 1024, nullptr),
         RLK_ERR_INVALID_ARG, false, "bwd f32: shifted overlap");
  expect(rlk_logp_backward_f32(f, 1024, t, nullptr, g, g, 4, 1000, f, 1028, nullptr),
         RLK_ERR_INVALID_ARG, false, "bwd f32: same base, other stride");

  // fused path
  const size_t ws = rlk_linear_logp_workspace_size(300, 1000, 64);
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, 300, 1000, 64, f, nullptr, g, ws, nullptr),
         RLK_OK, true, "fused: valid");
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, 300, 1000, 64, f, nullptr, g, ws - 1, nullptr),
         RLK_ERR_INVALID_ARG, false, "fused: workspace too small");
  expect(rlk_linear_logp(x, int64_t(1) << 22, x, 64, t, nullptr, 300, 1000, 64, f, nullptr, g, ws,
                         nullptr),
         RLK_ERR_UNSUPPORTED, false, "fused: ld_h at 2^22");
  expect(rlk_linear_logp(x, (int64_t(1) << 22) - 8, x, (int64_t(1) << 22) - 8, t, nullptr, 3,
                         260, (int64_t(1) << 22) - 8, f, nullptr, g,
                         rlk_linear_logp_workspace_size(3, 260, 0), nullptr),
         RLK_OK, true, "fused: largest H");
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, kMaxN, int64_t(1) << 28, 64, f, nullptr, g,
                         SIZE_MAX, nullptr),
         RLK_ERR_UNSUPPORTED, false, "fused: tile count beyond 2^23");
  // a launch holds fewer than 2^32 work-items: fewer than 2^23 tiles of 512
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, 14122 * 256, 151936, 64, f, nullptr, g,
                         SIZE_MAX, nullptr),
         RLK_OK, true, "fused: 8388468 tiles (V = 151936)");
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, 14122 * 256 + 1, 151936, 64, f, nullptr, g,
                         SIZE_MAX, nullptr),
         RLK_ERR_UNSUPPORTED, false, "fused: 8389062 tiles (V = 151936)");
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, (int64_t(1) << 24) - 256, 32768, 64, f, nullptr,
                         g, SIZE_MAX, nullptr),
         RLK_OK, true, "fused: 2^23 - 128 tiles");
  expect(rlk_linear_logp(x, 64, x, 64, t, nullptr, int64_t(1) << 24, 32768, 64, f, nullptr, g,
                         SIZE_MAX, nullptr),
         RLK_ERR_UNSUPPORTED, false, "fused: 2^23 tiles");
  expect(rlk_logp_backward(nullptr, 0, x, 64, x, 64, 64, t, nullptr, f, f, int64_t(1) << 24, 32768,
                           g, 32768, nullptr),
         RLK_ERR_UNSUPPORTED, false, "fused bwd: 2^23 tiles");
  expect(rlk_linear_logp_with_logits(x, 64, x, 64, t, nullptr, 300, 1000, 64, f, nullptr, g, 1000,
                                     at(A + 0x30000000), ws, nullptr),
         RLK_OK, true, "kept logits: valid");
  expect(rlk_logp_backward(nullptr, 0, x, 64, x, 64, 64, t, nullptr, f, f, 300, 1000, g, 1000,
                           nullptr),
         RLK_OK, true, "fused bwd: valid");
  const size_t wsg = rlk_linear_logp_param_grads_workspace_size(300, 1000, 64);
  expect(rlk_linear_logp_param_grads(x, 64, x, 64, t, nullptr, f, f, 300, 1000, 64, g, 64, g, 64,
                                     g, wsg, nullptr),
         RLK_OK, true, "param grads: valid");
  expect(rlk_linear_logp_param_grads(x, 64, x, 64, t, nullptr, f, f, 300, 1000, 64, nullptr, 0,
                                     nullptr, 0, g, wsg, nullptr),
         RLK_ERR_INVALID_ARG, false, "param grads: no output");
  expect(rlk_linear_logp_param_grads(x, 64, x, 64, t, nullptr, f, f, 0, 1000, 64, nullptr, 0, g,
                                     64, nullptr, 0, nullptr),
         RLK_OK, true, "param grads: N = 0 clears grad_weight");
  // the largest gradient launch: ceil(H/256) * ceil(N/256) (rounded up to 8)
  // + ceil(H/256) * (chunk tiles) workgroups, fewer than 2^23
  expect(rlk_linear_logp_param_grads(x, int64_t(1) << 19, x, int64_t(1) << 19, t, nullptr, f, f,
                                     (int64_t(1) << 20) - 1280, 1000, int64_t(1) << 19, g,
                                     int64_t(1) << 19, g, int64_t(1) << 19, g, SIZE_MAX, nullptr),
         RLK_OK, true, "param grads: 8386560 workgroups");
  expect(rlk_linear_logp_param_grads(x, int64_t(1) << 19, x, int64_t(1) << 19, t, nullptr, f, f,
                                     (int64_t(1) << 20) - 1024, 1000, int64_t(1) << 19, g,
                                     int64_t(1) << 19, g, int64_t(1) << 19, g, SIZE_MAX, nullptr),
         RLK_ERR_UNSUPPORTED, false, "param grads: 2^23 workgroups");
  // the row kernels loop over rows past their grid: any N < 2^31 launches
  expect(rlk_logp_selected(x, 1024, t, nullptr, kMaxN, 1024, f, nullptr, nullptr), RLK_OK, true,
         "logits: N = 2^31 - 1");
  expect(rlk_linear_logp_param_grads_from_logits(f, 1000, x, 64, x, 64, t, nullptr, f, f, 300,
                                                 1000, 64, g, 64, g, 64, g, wsg, nullptr),
         RLK_OK, true, "param grads from logits: valid");
  expect(rlk_linear_logp_param_grads_from_logits(nullptr, 1000, x, 64, x, 64, t, nullptr, f, f,
                                                 300, 1000, 64, g, 64, g, 64, g, wsg, nullptr),
         RLK_ERR_INVALID_ARG, false, "param grads from logits: no logits");

  // per-token losses
  expect(rlk_token_losses(f, f, nullptr, f, nullptr, 16, 0.2f, 0.2f, 0.0f, g, nullptr, nullptr,
                          nullptr, nullptr),
         RLK_OK, true, "losses: valid");
  expect(rlk_token_losses(f, f, nullptr, f, nullptr, 16, 1.5f, 0.2f, 0.0f, g, nullptr, nullptr,
                          nullptr, nullptr),
         RLK_ERR_INVALID_ARG, false, "losses: eps_lo >= 1");

  printf("%s (%d launches reached)\n", fails == 0 ? "sanitized validation ok" : "FAILED",
         g_launches);
  return fails == 0 ? 0 : 1;
}
