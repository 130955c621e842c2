/* Host-side driver for the sanitizer build of the C ABI's validation layer:
 * every entry point called with arguments it must refuse before any launch,
 * the status strings, and the timing hooks with nothing recorded. Prints one
 * line per failed expectation and exits non-zero if any failed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "prefill_attn.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    int got_ = (call);                                                                  \
    if (got_ != (want)) {                                                               \
      printf("FAIL %s:%d %s -> %d, want %d\n", __FILE__, __LINE__, #call, got_, (want)); \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main(void) {
  const uint16_t* P = (const uint16_t*)(uintptr_t)0x100000;  /* aligned, never dereferenced */
  float* F = (float*)(uintptr_t)0x100000;
  int32_t* I = (int32_t*)(uintptr_t)0x100000;
  void* W = (void*)(uintptr_t)0x100000;

  for (int s = -6; s <= 1; ++s)
    if (pa_status_string(s) == NULL || strlen(pa_status_string(s)) == 0) { printf("FAIL status %d\n", s); ++failures; }

  /* dense, all three mask forms and the allocation-free entry */
  EXPECT(prefill_attn_dense(NULL, 64, 4, P, P, 256, 2, 128, P, 256, 0.125f, F, W, 1 << 20, NULL), PA_EINVAL);
  EXPECT(prefill_attn_dense(P, 64, 3, P, P, 256, 2, 128, P, 256, 0.125f, F, W, 1 << 20, NULL), PA_EINVAL);
  EXPECT(prefill_attn_dense(P, 64, 4, P, P, 256, 2, 128, P, 255, 0.125f, F, W, 1 << 20, NULL), PA_EINVAL);
  EXPECT(prefill_attn_dense(P, 64, 4, P, P, 256, 2, 96, P, 256, 0.125f, F, W, 1 << 20, NULL), PA_EUNSUPPORTED);
  EXPECT(prefill_attn_dense(P, 64, 4, P, P, (1 << 22) - 4095, 2, 128, P, 1 << 22, 0.125f, F, W, 1 << 20, NULL),
         PA_EUNSUPPORTED);
  EXPECT(prefill_attn_dense(P, 64, 4, P, P, 256, 2, 128, P, 256, 0.125f, F, NULL, 0, NULL), PA_EWORKSPACE);
  EXPECT(prefill_attn_dense(P, 64, 4, P, P, 256, 2, 128, P, 256, 0.125f, F, W, 1, NULL), PA_EWORKSPACE);
  EXPECT(prefill_attn_dense_bits(P, 64, 4, P, P, 256, 2, 128, (const uint32_t*)P, 7, 0.125f, F, W, 1 << 20, NULL),
         PA_EINVAL);
  EXPECT(prefill_attn_dense_causal(P, 64, 200, 4, P, P, 256, 2, 128, NULL, 0.125f, F, W, 1 << 20, NULL),
         PA_EINVAL);
  EXPECT(prefill_attn_dense_causal(P, 64, 0, 4, P, P, 256, 2, 128, NULL, -1.0f, F, W, 1 << 20, NULL), PA_EINVAL);
  EXPECT(prefill_attn_dense_noalloc(P, 64, 4, P, P, 200000, 4, 128, P, 200000, 0.125f, F, NULL), PA_ESCRATCH);
  EXPECT(prefill_attn_dense_noalloc(P, 64, 4, P, P, 256, 2, 128, P, 100, 0.125f, F, NULL), PA_EINVAL);
  if (prefill_attn_dense_workspace(64, 256, 4, 2, 128) == 0) { printf("FAIL workspace size\n"); ++failures; }
  if (prefill_attn_dense_workspace(64, 256, 3, 2, 128) != 0) { printf("FAIL workspace size 0\n"); ++failures; }

  /* pooled index, selection, block-sparse */
  EXPECT(build_pooled_index(P, P, 0, 1, 128, 128, F, F, NULL), PA_EINVAL);
  EXPECT(build_pooled_index(P, P, 10, 1, 128, 48, F, F, NULL), PA_EUNSUPPORTED);
  EXPECT(build_pooled_index_ld(P, P, 1000, 2, 128, 128, 9, F, F, 8, NULL), PA_EINVAL);
  EXPECT(select_blocks(P, 256, 0, 4, 2, 128, F, 300, 128, 0.1f, 0.125f, I, I, NULL), PA_EINVAL);
  EXPECT(select_blocks(P, 256, 0, 4, 2, 128, F, 256, 128, -0.1f, 0.125f, I, I, NULL), PA_EINVAL);
  EXPECT(select_blocks(P, 16 * 8192 + 16, 0, 4, 2, 128, F, 16 * 8192 + 16, 16, 0.1f, 0.125f, I, I, NULL),
         PA_EUNSUPPORTED);
  EXPECT(select_blocks_ld(P, 256, 744, 4, 2, 128, F, 8, 1000, 128, 0.1f, 0.125f, 0, -1, 0, I, I, NULL), PA_EINVAL);
  EXPECT(prefill_attn_blocksparse(P, 256, 0, 4, P, P, 256, 2, 128, F, F, 48, I, I, 0.1f, F, W, 1 << 20, NULL),
         PA_EUNSUPPORTED);
  EXPECT(prefill_attn_blocksparse(P, 256, 0, 4, P, P, 256, 2, 128, F, F, 64, I, I, 0.1f, F, W, 0, NULL),
         PA_EWORKSPACE);
  EXPECT(prefill_attn_blocksparse_ld(P, 256, 744, 4, P, P, 1000, 2, 128, F, F, 7, 128, I, I, 0.1f, F, W, 1 << 30,
                                     NULL), PA_EINVAL);
  if (prefill_attn_blocksparse_workspace(0, 2, 128) != 0) { printf("FAIL bs workspace 0\n"); ++failures; }
  EXPECT(fold_keep_mask(I, 8, I, 16, 100, 115, 4, 3, (uint16_t*)P, 116, NULL), PA_EINVAL);
  EXPECT(fold_keep_mask(I, 8, I, 16, 100, 116, 0, 3, (uint16_t*)P, 116, NULL), PA_EINVAL);

  /* timing hooks with nothing recorded */
  double ms = -1.0;
  int64_t n = -1;
  EXPECT(pa_timing_read("nope", &ms, &n), PA_EINVAL);
  EXPECT(pa_timing_read(NULL, &ms, &n), PA_EINVAL);
  EXPECT(pa_timing_enable(1), PA_OK);
  EXPECT(pa_timing_reset(), PA_OK);
  EXPECT(pa_timing_read("attn_dense", &ms, &n), PA_OK);
  if (n != 0 || ms != 0.0) { printf("FAIL timing totals\n"); ++failures; }
  EXPECT(pa_timing_enable(0), PA_OK);

  printf("%d failures\n", failures);
  return failures != 0;
}
