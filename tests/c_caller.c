/* A plain C99 caller of the library: include/rlk.h must compile as C and
 * librlk.so must link and answer without C++ or Python in between.  Only
 * entry points that need no GPU are called: build information, status
 * strings, workspace sizes, and argument validation (which rejects before
 * any launch). */
#include <stdio.h>
#include <string.h>

#include "rlk.h"

static int fails = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAIL %s\n", what);
    fails++;
  }
}

int main(void) {
  const char* info = rlk_build_info();
  expect(info != NULL && strstr(info, "gfx950") != NULL, "build info names gfx950");
  expect(strcmp(rlk_status_string(RLK_OK), "RLK_OK") == 0, "status string of RLK_OK");
  expect(strcmp(rlk_status_string(RLK_ERR_UNSUPPORTED), "RLK_ERR_UNSUPPORTED") == 0,
         "status string of RLK_ERR_UNSUPPORTED");
  expect(rlk_linear_logp_workspace_size(8192, 128256, 4096) > 0, "fused workspace size");
  expect(rlk_linear_logp_param_grads_workspace_size(2048, 151936, 5120) > 0,
         "gradient workspace size");
  /* fake, never dereferenced device addresses: validation rejects first */
  const void* a16 = (const void*)0x10000;
  float* f16 = (float*)0x10000;
  expect(rlk_logp_selected(a16, 1024, (const int64_t*)a16, NULL, 0, 1024, f16, NULL, NULL) ==
             RLK_OK, "N == 0 is a no-op");
  expect(rlk_logp_selected(NULL, 1024, (const int64_t*)a16, NULL, 4, 1024, f16, NULL, NULL) ==
             RLK_ERR_INVALID_ARG, "missing logits");
  expect(rlk_logp_selected(a16, 1028, (const int64_t*)a16, NULL, 4, 1024, f16, NULL, NULL) ==
             RLK_ERR_UNSUPPORTED, "ld % 8");
  expect(rlk_logp_backward_f32(f16, 1024, (const int64_t*)a16, NULL, f16, f16, 4, 1000, NULL,
                               1024, NULL) == RLK_ERR_INVALID_ARG, "missing gradient output");
  printf("%s\n", fails == 0 ? "c caller ok" : "c caller failed");
  return fails == 0 ? 0 : 1;
}
