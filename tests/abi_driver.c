/* Host-side exercise of the C ABI (include/lora4.h) for a sanitized build of
 * the library: every entry point is called with arguments its validation
 * must refuse (and the size queries with valid and invalid ones), so only
 * host code runs and no GPU is needed. Built and run by
 * tests/test_abi_sanitized.py with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code of both; prints "ok" and exits
 * 0 when every status is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lora4.h"

static int failures = 0;

static void expect(const char *what, long got, long want) {
  if (got != want) {
    printf("FAIL %s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}

static void expect_nonzero(const char *what, size_t got) {
  if (got == 0) {
    printf("FAIL %s: got 0\n", what);
    ++failures;
  }
}

int main(void) {
  /* fake, 256-byte aligned device addresses: validation never dereferences */
  void *P = (void *)(uintptr_t)0x100000;
  void *Q = (void *)(uintptr_t)0x200000;
  void *MIS = (void *)(uintptr_t)0x100008; /* 8-byte aligned only */
  const uint16_t *X = (const uint16_t *)P;
  uint16_t *Y = (uint16_t *)Q;
  lora4_W W;
  memset(&W, 0, sizeof(W));
  W.format = LORA4_NF4;
  W.block = 64;
  W.N = 1024;
  W.K = 1024;
  W.groups = 1;
  W.codes = (const uint8_t *)P;
  W.scales = P;

  /* size queries */
  expect_nonzero("workspace fwd", lora4_workspace_bytes(0, &W, 256, 16));
  expect_nonzero("workspace bwd", lora4_workspace_bytes(1, &W, 256, 16));
  expect("workspace bad which", (long)lora4_workspace_bytes(2, &W, 256, 16), 0);
  expect("workspace bad rank", (long)lora4_workspace_bytes(0, &W, 256, 0), 0);
  expect("workspace null W", (long)lora4_workspace_bytes(0, NULL, 256, 16), 0);
  expect_nonzero("workspace multi", lora4_workspace_bytes_multi(0, &W, 4, 256, 16));
  expect("workspace multi bad", (long)lora4_workspace_bytes_multi(0, &W, 0, 256, 16), 0);
  expect_nonzero("packed codes", lora4_packed_bytes(LORA4_MXFP4, 100, 96, 0));
  expect_nonzero("packed scales", lora4_packed_bytes(LORA4_NVFP4, 100, 96, 1));
  expect("packed bad K", (long)lora4_packed_bytes(LORA4_NF4, 100, 96, 0), 0);
  expect("packed bad part", (long)lora4_packed_bytes(LORA4_NF4, 64, 64, 3), 0);
  expect("packed bad format", (long)lora4_packed_bytes(7, 64, 64, 0), 0);
  expect_nonzero("loftq workspace", lora4_loftq_workspace_bytes(256, 512, 16));
  expect("loftq workspace bad", (long)lora4_loftq_workspace_bytes(16, 512, 16), 0);

  /* forward / backward refusals */
  const size_t ws = (size_t)1 << 30;
  expect("fwd null W", lora4_forward(NULL, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL),
         LORA4_ERR_NULL);
  W.format = 9;
  expect("fwd format", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL),
         LORA4_ERR_FORMAT);
  W.format = LORA4_NF4;
  W.block = 32;
  expect("fwd block", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL),
         LORA4_ERR_FORMAT);
  W.block = 64;
  W.K = 96;
  expect("fwd K", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL), LORA4_ERR_SHAPE);
  W.K = 1024;
  expect("fwd rank", lora4_forward(&W, X, 16, X, X, 0, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL), LORA4_ERR_SHAPE);
  expect("fwd misaligned X", lora4_forward(&W, (const uint16_t *)MIS, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q,
                                           ws, NULL),
         LORA4_ERR_ALIGN);
  expect("fwd small workspace", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, 16, NULL),
         LORA4_ERR_WORKSPACE);
  expect("fwd null workspace", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, NULL, ws, NULL),
         LORA4_ERR_WORKSPACE);
  expect("fwd offsets without groups",
         lora4_forward(&W, X, 16, X, X, 16, 2.f, (const int64_t *)P, Y, NULL, NULL, NULL, Q, ws, NULL),
         LORA4_ERR_SHAPE);
  W.groups = 4;
  expect("fwd groups without offsets", lora4_forward(&W, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL),
         LORA4_ERR_NULL);
  W.groups = 1;
  expect("bwd null dA", lora4_backward(&W, X, X, 16, X, X, 16, 2.f, NULL, NULL, Y, NULL, Y, Q, ws, NULL),
         LORA4_ERR_NULL);
  expect("bwd nonfinite s", lora4_backward(&W, X, X, 16, X, X, 16, 1.f / 0.f, NULL, NULL, Y, Y, Y, Q, ws, NULL),
         LORA4_ERR_SHAPE);
  expect("multi adapters on grouped base",
         lora4_forward_multi(&W, 0, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, Q, ws, NULL), LORA4_ERR_SHAPE);
  expect("multi bwd no offsets",
         lora4_backward_multi(&W, 3, X, X, 16, X, X, 16, 2.f, NULL, NULL, Y, Y, Y, Q, ws, NULL), LORA4_ERR_NULL);
  expect("noalloc rank", lora4_forward_noalloc(&W, X, 16, X, X, 300, 2.f, NULL, Y, NULL, NULL, NULL, NULL),
         LORA4_ERR_SHAPE);
  expect("noalloc null W", lora4_forward_noalloc(NULL, X, 16, X, X, 16, 2.f, NULL, Y, NULL, NULL, NULL, NULL),
         LORA4_ERR_NULL);

  /* MX-native forward */
  expect("mx on nf4", lora4_forward_mx(&W, X, 16, X, X, 16, 2.f, Y, NULL, Q, ws, NULL), LORA4_ERR_FORMAT);
  expect("mx workspace on nf4", (long)lora4_workspace_bytes_mx(&W, 16, 16), 0);

  /* packers */
  expect("pack nf4 K", quant_pack_nf4(X, 64, 96, 0, (uint8_t *)Q, Q, NULL, NULL), LORA4_ERR_SHAPE);
  expect("pack nf4 dq null", quant_pack_nf4(X, 64, 64, 1, (uint8_t *)Q, Q, NULL, NULL), LORA4_ERR_NULL);
  expect("pack mxfp4 align", quant_pack_mxfp4((const uint16_t *)MIS, 64, 64, (uint8_t *)Q, (uint8_t *)Q, NULL),
         LORA4_ERR_ALIGN);
  expect("pack nvfp4 K", quant_pack_nvfp4(X, 64, 48, (uint8_t *)Q, (uint8_t *)Q, NULL), LORA4_ERR_SHAPE);
  expect("pack mxfp8 K", quant_pack_mxfp8(X, 16, 40, (uint8_t *)Q, (uint8_t *)Q, NULL), LORA4_ERR_SHAPE);
  expect("pack mxfp8 M 0", quant_pack_mxfp8(X, 0, 64, (uint8_t *)Q, (uint8_t *)Q, NULL), LORA4_OK);
  expect("import format", lora4_import_rowmajor(8, 64, 64, 1, (const uint8_t *)P, P, (uint8_t *)Q, Q, NULL),
         LORA4_ERR_FORMAT);
  expect("import align", lora4_import_rowmajor(1, 64, 64, 1, (const uint8_t *)MIS, P, (uint8_t *)Q, Q, NULL),
         LORA4_ERR_ALIGN);

  /* LoftQ */
  expect("loftq iters", lora4_loftq_init(X, 256, 512, 16, 0, 1.f, 0, (uint8_t *)Q, Q, NULL, Y, Y, Q, ws, NULL),
         LORA4_ERR_SHAPE);
  expect("loftq null", lora4_loftq_init(NULL, 256, 512, 16, 5, 1.f, 0, (uint8_t *)Q, Q, NULL, Y, Y, Q, ws, NULL),
         LORA4_ERR_NULL);

  /* helpers */
  for (int s = -8; s <= 0; ++s)
    if (!lora4_status_string((lora4_status)s) || !strcmp(lora4_status_string((lora4_status)s), "unknown status"))
      expect("status string", s, 1);
  expect("timing enable", lora4_timing_enable(0), LORA4_OK);
  expect("timing collect (empty)", lora4_timing_collect(NULL, 0), 0);
  if (!strstr(lora4_version(), "gfx950")) expect("version", 0, 1);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
