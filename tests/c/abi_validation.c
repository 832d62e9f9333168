/* Host-side validation of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (see test_abi_sanitized.py).
 * Every call below has an invalid argument, or is a host-only query, so the
 * library returns before any HIP call: no GPU is needed.  Device pointers are
 * stand-in addresses that are never dereferenced on the host.
 * Exit status 0 when every status and error text is as expected. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "oscar.h"

static int failures = 0;

#define EXPECT(call, want)                                                          \
  do {                                                                              \
    int st_ = (call);                                                               \
    if (st_ != (want)) {                                                            \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, \
              st_, (want), oscar_last_error());                                     \
      ++failures;                                                                   \
    } else if ((want) != OSCAR_OK && oscar_last_error()[0] == '\0') {               \
      fprintf(stderr, "line %d: %s: no error text\n", __LINE__, #call);             \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

static void *dev(uintptr_t a) { return (void *)a; }

static oscar_cache cache(void) {
  oscar_cache c;
  memset(&c, 0, sizeof c);
  c.num_kv_heads = 8;
  c.head_dim = 128;
  c.group_size = 64;
  c.page_size = 16;
  c.int2_pool = (uint8_t *)dev(0x100000);
  c.num_int2_pages = 100;
  c.bf16_k_pool = (uint16_t *)dev(0x200000);
  c.bf16_v_pool = (uint16_t *)dev(0x300000);
  c.num_bf16_pages = 40;
  return c;
}

static oscar_decode_args args(void) {
  oscar_decode_args a;
  memset(&a, 0, sizeof a);
  a.batch = 2;
  a.num_q_heads = 32;
  a.hist_pages = (const int32_t *)dev(0x400000);
  a.hist_stride = 10;
  a.hist_len = (const int32_t *)dev(0x500000);
  a.bf16_pages = (const int32_t *)dev(0x600000);
  a.bf16_stride = 20;
  a.bf16_len = (const int32_t *)dev(0x700000);
  a.max_hist_len = 100;
  return a;
}

int main(void) {
  size_t bytes = 0;
  int32_t ns = 0, pps = 0, kind = 0;
  oscar_cache c = cache();
  oscar_decode_args a = args();
  int32_t head_map[32];

  /* host-only queries with valid arguments */
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_OK);
  if (bytes == 0 || oscar_decode_workspace_bytes(&c, &a) != bytes) {
    fprintf(stderr, "workspace bytes %zu vs %zu\n", bytes, oscar_decode_workspace_bytes(&c, &a));
    ++failures;
  }
  /* the size query reports invalid arguments as 0 bytes, with an error text */
  a.batch = 0;
  if (oscar_decode_workspace_bytes(&c, &a) != 0 || oscar_last_error()[0] == '\0') {
    fprintf(stderr, "workspace bytes of invalid arguments\n");
    ++failures;
  }
  a = args();
  if (oscar_decode_workspace_bytes(NULL, &a) != 0 || oscar_decode_workspace_bytes(&c, NULL) != 0) {
    fprintf(stderr, "workspace bytes of NULL descriptors\n");
    ++failures;
  }
  EXPECT(oscar_decode_plan(&c, &a, &ns, &pps, &bytes, &kind), OSCAR_OK);
  if (kind != OSCAR_INT2_MFMA) { fprintf(stderr, "AUTO resolved to %d\n", kind); ++failures; }
  if (oscar_record_bytes(128, 64) != 1280 || oscar_record_bytes(100, 64) != 0) {
    fprintf(stderr, "record bytes\n");
    ++failures;
  }

  /* cache descriptor errors */
  c.head_dim = 96;   EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EUNSUPPORTED); c = cache();
  c.group_size = 48; EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EUNSUPPORTED); c = cache();
  c.page_size = 32;  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); c = cache();
  c.num_kv_heads = 0; EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); c = cache();
  c.status = (uint32_t *)dev(0x1002);   /* status word not 4-byte aligned */
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL);
  EXPECT(oscar_demote_pack(&c, 2, (const int32_t *)dev(0x800000), (const int32_t *)dev(0x800100),
                           (const float *)dev(0x900000), NULL, (const float *)dev(0x900000),
                           (const float *)dev(0x900000), NULL), OSCAR_EINVAL);
  c = cache();
  EXPECT(oscar_decode_plan(NULL, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL);
  EXPECT(oscar_decode_plan(&c, NULL, NULL, NULL, &bytes, NULL), OSCAR_EINVAL);

  /* argument errors */
  a.batch = 0;            EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.num_q_heads = 12;     EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.num_q_heads = 512;    EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.hist_stride = 6;      EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.max_hist_len = -1;    EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.sm_scale = -1.f;      EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.int2_kernel = 9;      EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.phases = 8;           EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.flags = 2;            EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL); a = args();
  a.num_q_heads = 24;     EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EUNSUPPORTED); a = args();
  for (int h = 0; h < 32; ++h) head_map[h] = h % 8;   /* valid: 4 q heads per KV head */
  a.kv_head_of_q = head_map;
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_OK);
  head_map[0] = 8;                                    /* out of range */
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL);
  head_map[0] = 1;                                    /* unequal group sizes */
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_EINVAL);
  a = args();

  /* launching calls, each with one invalid argument: nothing is enqueued */
  EXPECT(oscar_decode_plan(&c, &a, NULL, NULL, &bytes, NULL), OSCAR_OK);
  EXPECT(oscar_decode_attn(&c, &a, (const uint16_t *)dev(0x800000), (const float *)dev(0x900000),
                           dev(0xA00000), bytes - 1, NULL), OSCAR_EWORKSPACE);
  EXPECT(oscar_decode_attn(&c, &a, NULL, (const float *)dev(0x900000), dev(0xA00000), bytes, NULL),
         OSCAR_EINVAL);
  EXPECT(oscar_merge(&c, &a, dev(0xA00000), bytes, NULL, NULL, NULL, NULL), OSCAR_EINVAL);
  EXPECT(oscar_merge(&c, &a, dev(0xA00000), 16, NULL, (float *)dev(0xB00000), NULL, NULL),
         OSCAR_EWORKSPACE);
  EXPECT(oscar_write_bf16(&c, -1, NULL, NULL, NULL, NULL), OSCAR_EINVAL);
  EXPECT(oscar_write_bf16(&c, 3, NULL, (const uint16_t *)dev(0x800000), (const uint16_t *)dev(0x800000),
                          NULL), OSCAR_EINVAL);
  EXPECT(oscar_demote_pack(&c, 2, (const int32_t *)dev(0x800000), (const int32_t *)dev(0x800100),
                           NULL, NULL, (const float *)dev(0x900000), (const float *)dev(0x900000), NULL),
         OSCAR_EINVAL);
  a.phases = OSCAR_PHASE_INT2;
  EXPECT(oscar_decode_step(&c, &a, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                           dev(0xA00000), bytes, NULL, NULL, NULL), OSCAR_EINVAL);
  a = args();

  /* the allocation-free step: argument errors, and a workspace larger than
     its static array, are rejected before any HIP call */
  {
    const int32_t *sl = (const int32_t *)dev(0x800000);
    const float *fp = (const float *)dev(0x900000);
    const uint16_t *tk = (const uint16_t *)dev(0xC00000);
    EXPECT(oscar_decode_step_noalloc(&c, &a, sl, sl, fp, fp, sl, tk, tk, tk, fp, fp, NULL, NULL, NULL),
           OSCAR_EINVAL);                                         /* out is NULL */
    EXPECT(oscar_decode_step_noalloc(&c, &a, NULL, sl, fp, fp, sl, tk, tk, tk, fp, fp,
                                     (float *)dev(0xB00000), NULL, NULL), OSCAR_EINVAL);
    oscar_decode_args big = args();
    big.batch = 256;                                          /* 256 x 100K: > 16 MiB */
    big.hist_stride = 6400;
    big.max_hist_len = 6400 * 16;
    EXPECT(oscar_decode_plan(&c, &big, NULL, NULL, &bytes, NULL), OSCAR_OK);
    if (bytes <= OSCAR_NOALLOC_WORKSPACE_BYTES) {
      fprintf(stderr, "expected a workspace above the static one, got %zu\n", bytes);
      ++failures;
    }
    EXPECT(oscar_decode_step_noalloc(&c, &big, sl, sl, fp, fp, sl, tk, tk, tk, fp, fp,
                                     (float *)dev(0xB00000), NULL, NULL), OSCAR_EWORKSPACE);
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi validation: all checks passed\n");
  return 0;
}
