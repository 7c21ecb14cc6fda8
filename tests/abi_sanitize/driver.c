/*
 * Host-side driver for the sanitizer build of libfa_attn.so's argument
 * checks.  Every call below carries at least one invalid argument, so the
 * library must return the documented status before touching any pointer or
 * the GPU.  The values are chosen to reach the int64 size arithmetic with
 * extreme inputs (huge B, H, N, strides, windows, head counts), which is
 * where signed overflow would hide; the library and this driver are built
 * with AddressSanitizer and UndefinedBehaviorSanitizer, aborting on the
 * first report.  Exit status 0 means every status matched and nothing was
 * reported.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fa_attn.h"

static int failures = 0;

#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const int got_ = (call);                                                      \
    if (got_ != (want)) {                                                         \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
              got_, (int)(want));                                                 \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

/* fake, 16-byte aligned addresses; never dereferenced */
#define P(i) ((void*)(uintptr_t)(0x10000u * (unsigned)((i) + 1)))

/* sizes the checks must reject as B, H or N (each is < 1, above INT32_MAX,
   or, as N, a head of more than 2 GiB at d >= 64) */
static const int64_t BAD[] = {INT64_MAX, INT64_MAX / 2, INT64_MAX / 128, (int64_t)1 << 62,
                              (int64_t)1 << 61, (int64_t)1 << 40, (int64_t)1 << 33,
                              (int64_t)INT32_MAX + 1, INT64_MIN, -1, 0};
#define NBAD ((int)(sizeof(BAD) / sizeof(BAD[0])))

int main(void) {
  int i, j;
  for (i = 0; i < NBAD; ++i) {
    const int64_t x = BAD[i];
    EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), x, 1, 16, 64, 0, 0.125f, FA_BF16, 0), FA_ERR_SHAPE);
    EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, x, 16, 64, 0, 0.125f, FA_BF16, 0), FA_ERR_SHAPE);
    EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, x, 64, 0, 0.125f, FA_BF16, 0), FA_ERR_SHAPE);
    if (x > 0) EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, x, 0, 0.125f, FA_BF16, 0), FA_ERR_UNSUPPORTED);
    for (j = 0; j < NBAD; ++j) {
      EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), x, BAD[j], 4096, 128, 1, 0.1f, FA_F16, 0), FA_ERR_SHAPE);
      EXPECT(attn_bwd(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), x, BAD[j],
                      4096, 128, 1, 0.1f, FA_BF16, P(9), (size_t)1 << 20, 0),
             FA_ERR_SHAPE);
    }
    EXPECT(attn_fwd_dv(P(0), P(1), P(2), P(3), P(4), 1, 1, x, 128, 64, 1, 0.1f, FA_BF16, 0), FA_ERR_SHAPE);
    EXPECT(attn_bwd_dv(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1, 1, x,
                       128, 64, 1, 0.1f, FA_BF16, P(9), (size_t)1 << 20, 0),
           FA_ERR_SHAPE);
    EXPECT(attn_bwd_noalloc(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1,
                            1, x, 128, 1, 0.1f, FA_BF16, 0),
           FA_ERR_SHAPE);
    EXPECT(attn_fwd_window(P(0), P(1), P(2), P(3), P(4), 1, 1, x, 64, 5, 0.1f, FA_BF16, 0), FA_ERR_SHAPE);
    EXPECT(attn_fwd_kv_outer(P(0), P(1), P(2), P(3), P(4), x, 1, 4096, 128, 1, 0.1f, FA_BF16, P(9),
                             (size_t)1 << 30, 0),
           FA_ERR_SHAPE);
    if (x < 1) {
      EXPECT(attn_fwd_window(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, 64, x, 0.1f, FA_BF16, 0), FA_ERR_WINDOW);
      EXPECT(attn_bwd_window(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1, 1,
                             16, 64, x, 0.1f, FA_BF16, P(9), (size_t)1 << 20, 0),
             FA_ERR_WINDOW);
    }
    /* workspace queries return 0 for invalid sizes */
    if (attn_bwd_workspace_bytes(x, 16, 4096, 128, FA_BF16) != 0) ++failures;
    if (attn_bwd_block_sparse_workspace_bytes(1, 1, x, 128, FA_BF16) != 0) ++failures;
    if (attn_fwd_kv_outer_workspace_bytes(x, 1, 4096, 128, FA_BF16) != 0) ++failures;
  }
  /* strides the checks must reject: negative, not a multiple of 16 bytes,
     a row stride below d, rows of one head spanning 2 GiB, products that would
     overflow int64, and output axes that overlap */
  {
    const int64_t good[3] = {16 * 64 * 128, 64 * 128, 128};
    const int64_t bad_any[] = {-8, INT64_MIN, 7, 12, INT64_MAX, INT64_MAX - 7};
    int64_t st[3];
    int a, k;
    for (a = 0; a < 3; ++a)
      for (k = 0; k < (int)(sizeof(bad_any) / sizeof(bad_any[0])); ++k) {
        st[0] = good[0], st[1] = good[1], st[2] = good[2];
        st[a] = bad_any[k];
        EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, st, good, good, 1, 0.1f,
                                FA_BF16, 0),
               FA_ERR_STRIDE);
        EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, good, st, good, 1, 0.1f,
                                FA_BF16, 0),
               FA_ERR_STRIDE);
        EXPECT(attn_bwd_strided(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 2,
                                16, 64, 128, good, st, 1, 0.1f, FA_BF16, P(9), (size_t)1 << 30, 0),
               FA_ERR_STRIDE);
      }
    st[0] = good[0], st[1] = good[1], st[2] = 64;  /* rows closer than d */
    EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, st, good, good, 1, 0.1f, FA_BF16, 0),
           FA_ERR_STRIDE);
    st[2] = (int64_t)1 << 26;                      /* 63 rows of 128 MB: past 2 GiB */
    EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, st, good, good, 1, 0.1f, FA_BF16, 0),
           FA_ERR_SHAPE);
    st[0] = good[0], st[1] = 128, st[2] = 128;     /* outputs: heads overlap rows */
    EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, good, good, st, 1, 0.1f, FA_BF16, 0),
           FA_ERR_STRIDE);
    EXPECT(attn_fwd_strided(P(0), P(1), P(2), P(3), P(4), 2, 16, 64, 128, 0, good, good, 1, 0.1f, FA_BF16, 0),
           FA_ERR_NULL);
  }
  /* block-sparse: mask axes that are neither 1 nor the full extent */
  for (i = 0; i < NBAD; ++i) {
    if (BAD[i] == 1) continue;
    EXPECT(attn_fwd_block_sparse(P(0), P(1), P(2), P(3), P(4), 2, 3, 256, 64, (const uint8_t*)P(5),
                                 BAD[i], 1, 0, 0.1f, FA_BF16, 0),
           FA_ERR_SHAPE);
    EXPECT(attn_fwd_block_sparse(P(0), P(1), P(2), P(3), P(4), 2, 3, 256, 64, (const uint8_t*)P(5), 1,
                                 BAD[i], 0, 0.1f, FA_BF16, 0),
           FA_ERR_SHAPE);
  }
  EXPECT(attn_fwd_block_sparse(P(0), P(1), P(2), P(3), P(4), 1, 1, 256, 64, 0, 1, 1, 0, 0.1f, FA_BF16, 0),
         FA_ERR_NULL);
  /* a mask too large for a workgroup's tile list */
  EXPECT(attn_fwd_block_sparse(P(0), P(1), P(2), P(3), P(4), 1, 1, 64 * 2049, 64, (const uint8_t*)P(5),
                               1, 1, 0, 0.1f, FA_BF16, 0),
         FA_ERR_UNSUPPORTED);
  /* the split block-sparse backward grid (four workgroups per key block)
     must fit 2^31 - 1: B * H near 2^31 with one key block */
  EXPECT(attn_bwd_block_sparse(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1,
                               (int64_t)1 << 30, 16, 64, (const uint8_t*)P(9), 1, 1, 0, 0.1f, FA_BF16,
                               P(10), ~(size_t)0, 0),
         FA_ERR_SHAPE);
  /* allocation-free backward: more rows than its fixed scratch */
  EXPECT(attn_bwd_noalloc(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1, 1,
                          (int64_t)attn_bwd_noalloc_max_rows() + 1, 128, 1, 0.1f, FA_BF16, 0),
         FA_ERR_SCRATCH);
  /* scale, dtype, mask */
  EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, 64, 0, NAN, FA_BF16, 0), FA_ERR_SCALE);
  EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, 64, 0, INFINITY, FA_BF16, 0), FA_ERR_SCALE);
  EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, 64, 0, 0.1f, -5, 0), FA_ERR_DTYPE);
  EXPECT(attn_fwd(P(0), P(1), P(2), P(3), P(4), 1, 1, 16, 64, 9, 0.1f, FA_BF16, 0), FA_ERR_MASK);
  /* status strings, including codes outside the enum */
  for (i = -3; i < 40; ++i)
    if (fa_status_str(i) == 0) ++failures;
  if (fa_abi_version() < 1) ++failures;
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi sanitizer driver: all checks passed\n");
  return 0;
}
