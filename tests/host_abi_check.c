/* Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * against a host-instrumented build of the library (tests/test_host_sanitizers.py). Every call
 * fails its argument checks or is a no-op (B = 0, N = 0), so nothing is launched on any machine:
 * the pointers below stand in for device buffers and are never dereferenced. Prints one line per
 * failed expectation and exits with the number of failures. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tsc.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAILED: %s\n", what);
    ++failures;
  }
}

/* Stand-ins for device pointers: distinct, suitably aligned, never dereferenced. */
#define DPTR(n) ((void*)(uintptr_t)(0x10000u * (n)))

static int32_t sample(const void* logits, int32_t dtype, int64_t B, int64_t V, int64_t ld,
                      int64_t R, int32_t W, void* bits, int64_t bits_ld, int null_mask) {
  return tsc_sample_with_mask_bits(
      logits, dtype, B, V, ld, (null_mask & 1) ? NULL : (const float*)DPTR(2),
      (null_mask & 2) ? NULL : (const int32_t*)DPTR(3), (const float*)DPTR(4),
      (const float*)DPTR(5), (null_mask & 4) ? NULL : (const int32_t*)DPTR(6), R,
      (const uint64_t*)DPTR(7), (const uint64_t*)DPTR(8), W, (int32_t*)DPTR(9), (int8_t*)DPTR(10),
      (null_mask & 8) ? NULL : (int32_t*)DPTR(11), (float*)DPTR(12), (int32_t*)DPTR(13),
      (float*)DPTR(14), (uint8_t*)bits, bits_ld, NULL, 0, NULL);
}

int main(void) {
  const void* lg = DPTR(1);
  /* Argument checks of the sampler: each returns before any launch. */
  expect(sample(lg, 7, 4, 100, 100, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "bad dtype");
  expect(sample(lg, TSC_DTYPE_BF16, -1, 100, 100, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "B < 0");
  expect(sample(lg, TSC_DTYPE_BF16, 4, 0, 0, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "V = 0");
  expect(sample(lg, TSC_DTYPE_BF16, 4, 100, 99, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "ld < V");
  expect(sample(lg, TSC_DTYPE_BF16, 4, INT32_MAX, INT32_MAX, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "V too large");
  expect(sample(lg, TSC_DTYPE_BF16, 4, 100, 100, 5, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "R > B");
  expect(sample(lg, TSC_DTYPE_BF16, 0, 100, 100, 0, 16, NULL, 0, 0) == TSC_OK, "B = 0 is a no-op");
  expect(sample((const char*)lg + 1, TSC_DTYPE_BF16, 4, 100, 100, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "misaligned logits");
  expect(sample(NULL, TSC_DTYPE_F32, 4, 100, 100, 2, 16, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "null logits");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, NULL, 0, 1) == TSC_ERR_INVALID_ARGUMENT, "null temperature");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, NULL, 0, 2) == TSC_ERR_INVALID_ARGUMENT, "null top_k");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, NULL, 0, 4) == TSC_ERR_INVALID_ARGUMENT, "null optin_rows with R > 0");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, NULL, 0, 8) == TSC_ERR_INVALID_ARGUMENT, "null packed_ids with R > 0");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 0, NULL, 0, 0) == TSC_ERR_INVALID_ARGUMENT, "W = 0");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, TSC_MAX_PACKED_WIDTH + 1, NULL, 0, 0) == TSC_ERR_UNSUPPORTED, "W too wide");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, DPTR(15), 8, 0) == TSC_ERR_INVALID_ARGUMENT, "bits_ld too small");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, DPTR(15), 24, 0) == TSC_ERR_INVALID_ARGUMENT, "bits_ld not a multiple of 16");
  expect(sample(lg, TSC_DTYPE_F32, 4, 100, 100, 2, 16, (char*)DPTR(15) + 4, 16, 0) == TSC_ERR_INVALID_ARGUMENT, "misaligned bits");
  expect(tsc_workspace_size(4, 100, 2, 16, TSC_DTYPE_BF16) == 0, "workspace size");
  expect(tsc_support_bits_ld(0) == 0 && tsc_support_bits_ld(1) == 16 && tsc_support_bits_ld(129) == 32,
         "bitmask row sizes");
  expect(tsc_support_bits_ld(INT32_MAX - 16) % 16 == 0, "bitmask row size of the largest V");

  /* Replay and CSR argument checks. */
  expect(tsc_replay_logprob(lg, TSC_DTYPE_BF16, 4, 100, 100, (const float*)DPTR(2), (const int32_t*)DPTR(3),
                            (const int32_t*)DPTR(4), 0, NULL, NULL, 0, (const int32_t*)DPTR(5),
                            (float*)DPTR(6), NULL, (int8_t*)DPTR(7), NULL) == TSC_ERR_INVALID_ARGUMENT,
         "replay W = 0");
  expect(tsc_replay_logprob(lg, TSC_DTYPE_BF16, 4, 100, 100, (const float*)DPTR(2), (const int32_t*)DPTR(3),
                            (const int32_t*)DPTR(4), 16, NULL, (const uint8_t*)DPTR(8), 4,
                            (const int32_t*)DPTR(5), (float*)DPTR(6), NULL, (int8_t*)DPTR(7), NULL) ==
             TSC_ERR_INVALID_ARGUMENT,
         "replay bits_ld too small");
  expect(tsc_replay_logprob(lg, TSC_DTYPE_BF16, 0, 100, 100, NULL, NULL, NULL, 16, NULL, NULL, 0, NULL, NULL,
                            NULL, NULL, NULL) == TSC_OK,
         "replay N = 0 is a no-op");
  expect(tsc_support_csr(NULL, NULL, NULL, -1, 16, (int64_t*)DPTR(2), NULL, NULL, 0, NULL) ==
             TSC_ERR_INVALID_ARGUMENT,
         "csr R < 0");
  expect(tsc_support_csr((const int32_t*)DPTR(1), (const int32_t*)DPTR(3), NULL, 4, 16, NULL, NULL, NULL, 0,
                         NULL) == TSC_ERR_INVALID_ARGUMENT,
         "csr null offsets");
  expect(tsc_support_csr((const int32_t*)DPTR(1), (const int32_t*)DPTR(3), NULL, 4, TSC_MAX_PACKED_WIDTH + 1,
                         (int64_t*)DPTR(2), NULL, NULL, 0, NULL) == TSC_ERR_UNSUPPORTED,
         "csr W too wide");

  /* Host-side state and strings. */
  {
    const uint32_t prev = tsc_set_wait_limit(9);
    expect(tsc_set_wait_limit(0) == 9, "wait limit round trip");
    tsc_set_wait_limit(prev);
    const int32_t p = tsc_set_debug_poison(1);
    expect(tsc_set_debug_poison(p) == 1, "poison round trip");
  }
  for (int32_t c = -2; c < 8; ++c) expect(strlen(tsc_status_string(c)) > 0, "status string");
  expect(tsc_version() >= 100, "version");

  printf("host ABI checks: %d failure(s)\n", failures);
  return failures;
}
