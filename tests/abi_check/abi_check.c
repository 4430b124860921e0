/*
 * Host-only exercise of the C ABI's argument validation, built with AddressSanitizer (with the
 * library's host code also instrumented) and run by tests/test_abi_asan.py on a machine with or
 * without a GPU. Every call here is invalid in some way, so the library must return its status
 * before any HIP call: the fake device pointers below are never dereferenced. ASan reports any
 * out-of-bounds or use-after-free access in the validation and workspace-size code.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;
static int checks = 0;

#define P ((void*)0x100000)      /* fake 16-byte-aligned device address */
#define PM ((void*)0x100004)     /* misaligned */
#define FP ((float*)0x100000)
#define FPM ((float*)0x100004)

static void expect(const char* what, int got, int want, int line) {
  ++checks;
  if (got != want) {
    ++failures;
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect(#call, (int)(call), (int)(want), __LINE__)

static fa_status fwd(const void* q, void* o, float* lse, int B, int H, int N, int d, float scale,
                     int causal, int in_dt, int o_dt) {
  return fa_forward(q, P, P, o, lse, B, H, N, d, scale, causal, (fa_dtype)in_dt, (fa_dtype)o_dt,
                    NULL);
}

static fa_status bwd(const void* q, void* dq, int B, int H, int N, int d, float scale, int causal,
                     int in_dt, int o_dt, int g_dt, void* ws, size_t ws_bytes) {
  return fa_backward(q, P, P, P, P, FP, dq, P, P, B, H, N, d, scale, causal, (fa_dtype)in_dt,
                     (fa_dtype)o_dt, (fa_dtype)g_dt, ws, ws_bytes, NULL);
}

int main(void) {
  const float nan = __builtin_nanf("");
  const float inf = __builtin_inff();
  const size_t big = (size_t)1 << 40;

  /* Status strings: every code, and codes outside the enum. */
  for (int c = -3; c < 12; ++c) {
    const char* s = fa_status_string((fa_status)c);
    ++checks;
    if (s == NULL || strlen(s) == 0) {
      ++failures;
      fprintf(stderr, "fa_status_string(%d) is empty\n", c);
    }
  }

  /* Forward. */
  EXPECT(fwd(NULL, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(PM, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FPM, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 0, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, -1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 0, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 0, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, INT_MAX, INT_MAX, INT_MAX, 64, 0.1f, 0, FA_BF16, FA_BF16),
         FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, (1 << 24) + 1, 64, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 80, 0.1f, 0, FA_BF16, FA_BF16), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, nan, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, inf, 0, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, 0.1f, 2, FA_BF16, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, 0.1f, 0, 7, FA_BF16), FA_ERR_INVALID_ARG);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_F16), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_F32, FA_BF16), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(P, P, FP, 1, 1, 8, 256, 0.1f, 0, FA_F32, FA_F32), FA_ERR_UNSUPPORTED);

  /* fa_forward_kv. */
  EXPECT(fa_forward_kv(P, P, P, P, FP, 1, 1, 9, 8, 64, 0.1f, 1, FA_BF16, FA_BF16, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_kv(P, P, P, P, FP, 1, 1, 8, 0, 64, 0.1f, 0, FA_BF16, FA_BF16, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_kv(P, P, P, P, FP, 1, 1, 8, INT_MAX, 64, 0.1f, 0, FA_BF16, FA_BF16, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_kv(P, P, P, P, FP, 1, 1, 8, 8, 64, 0.1f, 0, FA_F32, FA_F32, NULL),
         FA_ERR_UNSUPPORTED);

  /* Dropout and block-sparse forwards. */
  EXPECT(fa_forward_dropout(P, P, P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16, -0.1f, 1, 0,
                            NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_dropout(P, P, P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16, 1.0f, 1, 0,
                            NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_dropout(P, P, P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16, nan, 1, 0,
                            NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_dropout(P, P, P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_F32, FA_F32, 0.1f, 1, 0,
                            NULL),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_forward_blocksparse(P, P, P, P, FP, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_BF16, NULL, 1,
                                NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_blocksparse(P, P, P, P, FP, 2, 3, 8, 64, 0.1f, 0, FA_BF16, FA_BF16,
                                (const uint8_t*)P, 5, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_forward_blocksparse(P, P, P, P, FP, 1, 1, 65537, 64, 0.1f, 0, FA_BF16, FA_BF16,
                                (const uint8_t*)P, 1, NULL),
         FA_ERR_UNSUPPORTED);

  /* Backward. */
  EXPECT(bwd(NULL, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, P, big),
         FA_ERR_INVALID_ARG);
  EXPECT(bwd(P, PM, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, P, big), FA_ERR_INVALID_ARG);
  EXPECT(bwd(P, P, 2, 3, 100, 64, nan, 1, FA_BF16, FA_F32, FA_F32, P, big), FA_ERR_INVALID_ARG);
  EXPECT(bwd(P, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, 9, P, big), FA_ERR_INVALID_ARG);
  EXPECT(bwd(P, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F16, P, big), FA_ERR_UNSUPPORTED);
  EXPECT(bwd(P, P, 2, 3, 100, 256, 0.1f, 1, FA_F32, FA_F32, FA_F32, P, big),
         FA_ERR_UNSUPPORTED);
  EXPECT(bwd(P, P, 2, 3, 100, 256, 0.1f, 1, FA_BF16, FA_F32, FA_F32, NULL, big),
         FA_ERR_WORKSPACE);
  EXPECT(bwd(P, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, NULL, big),
         FA_ERR_WORKSPACE);
  EXPECT(bwd(P, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, PM, big), FA_ERR_WORKSPACE);
  EXPECT(bwd(P, P, INT_MAX, 2, 3, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, P, big),
         FA_ERR_INVALID_ARG);
  {
    const size_t need = fa_backward_workspace_bytes(2, 3, 100, 64, FA_BF16, FA_F32);
    ++checks;
    if (need == 0) {
      ++failures;
      fprintf(stderr, "workspace size of a valid call is 0\n");
    }
    EXPECT(bwd(P, P, 2, 3, 100, 64, 0.1f, 1, FA_BF16, FA_F32, FA_F32, P, need - 1),
           FA_ERR_WORKSPACE);
  }
  EXPECT(fa_backward_kv(P, P, P, P, P, FP, P, P, P, 1, 1, 9, 8, 64, 0.1f, 1, FA_BF16, FA_F32,
                        FA_F32, P, big, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_backward_kv(P, P, P, P, P, FP, P, P, P, 1, 1, 8, 0, 64, 0.1f, 0, FA_BF16, FA_F32,
                        FA_F32, P, big, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_backward_dropout(P, P, P, P, P, FP, P, P, P, 1, 1, 8, 64, 0.1f, 0, FA_BF16, FA_F32,
                             FA_F32, 2.0f, 1, 0, P, big, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_backward_blocksparse(P, P, P, P, P, FP, P, P, P, 1, 1, 8, 64, 0.1f, 0, FA_BF16,
                                 FA_F32, FA_F32, NULL, 1, P, big, NULL),
         FA_ERR_INVALID_ARG);

  /* Workspace-size queries over extreme and rejected arguments: 0, never a crash. */
  {
    const int vals[] = {INT_MIN, -1, 0, 1, 7, 100, 65536, 1 << 24, INT_MAX};
    const int dims[] = {0, 16, 32, 64, 80, 96, 128, 256, INT_MAX};
    for (size_t i = 0; i < sizeof(vals) / sizeof(vals[0]); ++i)
      for (size_t j = 0; j < sizeof(dims) / sizeof(dims[0]); ++j)
        for (int dt = -1; dt < 4; ++dt) {
          const size_t a = fa_backward_workspace_bytes(vals[i], 3, vals[i], dims[j], (fa_dtype)dt,
                                                       FA_F32);
          const size_t b = fa_backward_kv_workspace_bytes(2, vals[i], 17, vals[i], dims[j],
                                                          (fa_dtype)dt, (fa_dtype)dt);
          const size_t c = fa_decode_workspace_bytes(1, vals[i], 1, vals[i], dims[j]);
          ++checks;
          /* A valid size is at most a few times the tensors' bytes (below 2^31 elements). */
          if (a > ((size_t)1 << 36) || b > ((size_t)1 << 36) || c > ((size_t)1 << 36)) {
            ++failures;
            fprintf(stderr, "implausible workspace size %zu %zu %zu\n", a, b, c);
          }
        }
  }

  /* Decoding. */
  EXPECT(fa_decode_forward(P, P, P, P, FP, 1, 1, 5, 100, 64, 0.1f, 1, FA_BF16, FA_BF16, P, big,
                           NULL),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_decode_forward(P, P, P, P, FP, 1, 1, 3, 2, 64, 0.1f, 1, FA_BF16, FA_BF16, P, big,
                           NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_decode_forward(P, P, P, P, FP, 1, 1, 1, 100, 64, 0.1f, 1, FA_BF16, FA_BF16, NULL,
                           big, NULL),
         FA_ERR_WORKSPACE);
  EXPECT(fa_decode_forward(P, P, P, P, FP, 1, 1, 1, 100, 32, 0.1f, 1, FA_BF16, FA_BF16, P, big,
                           NULL),
         FA_ERR_UNSUPPORTED);

  /* Allocation-free decoding: validation, and calls too large for its scratch. */
  EXPECT(fa_decode_forward_noalloc(NULL, P, P, P, FP, 1, 1, 1, 100, 64, 0.1f, 1, FA_BF16,
                                   FA_BF16, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_decode_forward_noalloc(P, P, P, P, FP, 64, 128, 4, 256, 128, 0.1f, 1, FA_BF16,
                                   FA_BF16, NULL),
         FA_ERR_WORKSPACE);
  EXPECT(fa_decode_forward_noalloc(P, P, P, P, FP, INT_MAX, 128, 4, 256, 128, 0.1f, 1, FA_BF16,
                                   FA_BF16, NULL),
         FA_ERR_INVALID_ARG);

  /* Timed backward: both events required, 16-bit inputs only, then fa_backward's checks. */
  EXPECT(fa_backward_timed(P, P, P, P, P, FP, P, P, P, 2, 3, 100, 64, 0.125f, 1, FA_BF16, FA_F32,
                           FA_F32, P, (size_t)1 << 30, NULL, P, NULL),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_backward_timed(P, P, P, P, P, FP, P, P, P, 2, 3, 100, 64, 0.125f, 1, FA_F32, FA_F32,
                           FA_F32, P, (size_t)1 << 30, NULL, P, P),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_backward_timed(P, P, P, P, P, FP, P, P, P, 2, 3, 100, 64, 0.125f, 1, FA_BF16, FA_F32,
                           FA_F32, NULL, 0, NULL, P, P),
         FA_ERR_WORKSPACE);

  if (failures) {
    fprintf(stderr, "%d of %d checks failed\n", failures, checks);
    return 1;
  }
  printf("abi_check: all %d checks passed\n", checks);
  return 0;
}
