/* The C ABI used from plain C (no C++, no torch): validation paths only, so
 * it runs without a GPU -- every call below is rejected before any HIP call.
 * Exit status 0 when every expectation holds; prints the first failure. */
#include <stdio.h>
#include <string.h>

#include "flashnorm.h"

static int fails = 0;

static void expect(int cond, const char* what) {
  if (!cond && fails++ == 0) fprintf(stderr, "FAILED: %s (last error: \"%s\")\n", what, fn_last_error());
}

int main(void) {
  void* x = (void*)0x1000;
  void* w = (void*)0x20000;
  void* y = (void*)0x40000;
  fn_step step = NULL;
  fn_call call;

  expect(fn_norm_proj(x, w, y, 4, 12, 16, 1e-6f, FN_BF16, NULL) == FN_ERR_SHAPE, "K % 8 rejected");
  expect(strstr(fn_last_error(), "K=12") != NULL, "error text names K");
  expect(fn_norm_proj(NULL, w, y, 4, 16, 16, 1e-6f, FN_BF16, NULL) == FN_ERR_NULL, "null x rejected");
  expect(fn_norm_proj(x, w, y, 4, 16, 16, -1.0f, FN_BF16, NULL) == FN_ERR_EPS, "negative eps rejected");
  expect(fn_norm_proj(x, w, x, 4, 16, 16, 1e-6f, FN_BF16, NULL) == FN_ERR_ALIAS, "y overlapping x rejected");
  expect(fn_norm_proj((void*)0x1002, w, y, 4, 16, 16, 1e-6f, FN_BF16, NULL) == FN_ERR_ALIGN, "misaligned x rejected");
  expect(fn_norm_proj(x, w, y, 4, 16, 16, 1e-6f, (fn_dtype)9, NULL) == FN_ERR_DTYPE, "unknown dtype rejected");
  expect(fn_norm_proj(x, w, y, 0, 16, 16, 1e-6f, FN_BF16, NULL) == FN_OK, "empty call is valid");
  expect(fn_norm_proj_swiglu(x, w, NULL, y, 4, 16, 16, 1e-6f, FN_BF16, NULL) == FN_ERR_NULL, "null W_up rejected");
  expect(fn_packed_weight_bytes(32, 16, FN_BF16) == 32 * 16 * 2, "packed size of one k-block x one column block");
  expect(fn_packed_weight_bytes(16, 16, FN_BF16) == 32 * 16 * 2, "a partial k-block is padded to a whole one");
  expect(fn_packed_weight_bytes(12, 16, FN_BF16) == 0, "packed size of a bad K is 0");
  expect(strlen(fn_status_string(FN_ERR_ALIAS)) > 0, "status strings");

  memset(&call, 0, sizeof call);
  call.kind = FN_CALL_NORM_PROJ;
  call.x = x;
  call.w_gate = w;
  call.y = y;
  call.M = 4;
  call.K = 12;
  call.N = 16;
  call.eps = 1e-6f;
  call.dt = FN_BF16;
  expect(fn_step_create(&call, 1, &step) == FN_ERR_SHAPE && step == NULL, "step validates its calls");
  expect(fn_step_create_grouped(&call, 1, &step) == FN_ERR_SHAPE && step == NULL, "grouped step validates its calls");
  expect(fn_step_num_kernels(NULL) == -1, "num_kernels of NULL");
  expect(fn_step_destroy(NULL) == FN_OK, "destroy NULL");
  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
