/* Plain C99 user of libfa.so: include/fa.h must compile as C, and every
 * argument error must be reported before any HIP call (no GPU needed).
 * Fake device addresses below are never dereferenced. */
#include <stdint.h>
#include <stdio.h>

#include "fa.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: got %d (%s), want %d\n", what, got, fa_status_string(got), want);
    ++failures;
  }
}

int main(void) {
  const uint16_t* a = (const uint16_t*)(uintptr_t)0x10000;   /* 16-B aligned */
  uint16_t* o = (uint16_t*)(uintptr_t)0x20000;
  float* lse = (float*)(uintptr_t)0x30000;
  void* ws = (void*)(uintptr_t)0x100000;                       /* 256-B aligned */
  const size_t wsb = fa_bwd_workspace_size(1, 2, 64, 128);

  if (fa_version() <= 0) { printf("FAIL version\n"); ++failures; }
  expect(fa_fwd(NULL, a, a, o, lse, 1, 2, 64, 64, 0.125f, 1, NULL), FA_ERR_NULL, "fwd null q");
  expect(fa_fwd(a, a, a, o, lse, 0, 2, 64, 64, 0.125f, 1, NULL), FA_ERR_SHAPE, "fwd B=0");
  expect(fa_fwd(a, a, a, o, lse, 1, 2, 64, 80, 0.125f, 1, NULL), FA_ERR_HEADDIM, "fwd d=80");
  expect(fa_fwd(a, a, a, (uint16_t*)(uintptr_t)0x20002, lse, 1, 2, 64, 64, 0.125f, 1, NULL),
         FA_ERR_ALIGN, "fwd misaligned o");
  expect(fa_fwd_f32(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 64, 1.f, 0, NULL), FA_ERR_NULL,
         "fwd_f32 null");
  expect(fa_bwd(a, a, a, a, a, lse, o, o, o, ws, wsb, 1, 2, 64, 96, 0.1f, 1, NULL),
         FA_ERR_HEADDIM, "bwd d=96");
  expect(fa_bwd(a, a, a, a, a, lse, o, o, o, NULL, wsb, 1, 2, 64, 128, 0.1f, 1, NULL),
         FA_ERR_WORKSPACE, "bwd no workspace");
  expect(fa_bwd(a, a, a, a, a, lse, o, o, o, ws, wsb - 1, 1, 2, 64, 128, 0.1f, 1, NULL),
         FA_ERR_WORKSPACE, "bwd small workspace");
  expect(fa_fwd_dropout(a, a, a, o, lse, 1, 2, 64, 128, 0.1f, 1, 1.5f, 7u, 0u, NULL),
         FA_ERR_DROPOUT, "dropout p=1.5");
  expect(fa_bwd_dropout(a, a, a, a, a, lse, o, o, o, ws, wsb, 1, 2, 64, 128, 0.1f, 1, -0.1f,
                        7u, 0u, NULL), FA_ERR_DROPOUT, "bwd dropout p<0");
  expect(fa_fwd_block_sparse(a, a, a, NULL, o, lse, 1, 2, 64, 128, 0.1f, 0, NULL), FA_ERR_NULL,
         "sparse null mask");
  expect(fa_linear_fwd(a, a, a, NULL, NULL, 0, 1, 2, 64, 128, 0.1f, NULL), FA_ERR_NULL,
         "linear null o");
  expect(fa_fp8_quantize(a, a, a, NULL, NULL, 0, 1, 2, 64, 128, NULL), FA_ERR_WORKSPACE,
         "fp8 null workspace");
  if (fa_bwd_workspace_size(1, 2, 64, 64) == 0) { printf("FAIL ws d=64\n"); ++failures; }
  if (fa_bwd_workspace_size(1, 2, 64, 96) != 0) { printf("FAIL ws d=96\n"); ++failures; }
  if (failures == 0) printf("C ABI checks passed\n");
  return failures == 0 ? 0 : 1;
}
