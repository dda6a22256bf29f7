/* Host-side checks of librkv run under AddressSanitizer and
 * UndefinedBehaviorSanitizer.
 *
 * The library's host code (schedule arithmetic, cache sizing, argument and
 * alignment validation, the decode split hint and the scratch-limit check of
 * the allocation-free decode) is built with host instrumentation only and
 * linked into this program.  Every call below is either pure host arithmetic
 * or is refused by validation before the library touches the device, so the
 * program needs no GPU; the fake device addresses it passes are never
 * dereferenced on the host, and a sanitizer report or a wrong status fails
 * it.  It prints "ok <count>" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rkv.h"

static int n_checks = 0;
static int n_failed = 0;

#define CHECK(cond)                                                    \
  do {                                                                 \
    ++n_checks;                                                        \
    if (!(cond)) {                                                     \
      ++n_failed;                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, \
              #cond);                                                  \
    }                                                                  \
  } while (0)

#define P(x) ((void *)(uintptr_t)(x))

static rkv_stride st(int32_t base, int64_t A) {
  rkv_stride s;
  s.base = base;
  s.double_after = A;
  return s;
}

/* A cache description with every buffer unset (the same defaults as the
 * Python host tests: two bf16 instances of 8 KV heads over 8192 positions,
 * stride 32, k = 8, 4-bit codes in groups of 32). */
static rkv_cache make_cache(int64_t n_inst, int32_t H, int64_t N, int32_t base) {
  rkv_cache c;
  memset(&c, 0, sizeof c);
  c.dtype = RKV_BF16;
  c.n_inst = n_inst;
  c.n_kv_heads = H;
  c.seq_len = N;
  c.head_dim = 128;
  c.stride = st(base, 0);
  c.k = 8;
  c.bits = 4;
  c.group = 32;
  return c;
}

static void set_buffers(rkv_cache *c, uintptr_t addr) {
  c->ref_idx = (uint16_t *)P(addr);
  c->codes_k = (uint8_t *)P(addr);
  c->codes_v = (uint8_t *)P(addr);
  c->scales = (uint16_t *)P(addr);
  c->ref_kv = P(addr);
}

/* Reference positions by walking every position: position j is a reference
 * when it is a multiple of the stride in force at j (the base, doubled each
 * time j reaches A, 2A, 4A, ... when A > 0).  Returns the count and writes
 * up to cap positions. */
static int64_t walk_refs(int64_t n, int32_t base, int64_t A, int64_t *pos, int64_t cap) {
  int64_t cnt = 0;
  for (int64_t j = 0; j < n; ++j) {
    int64_t s = base;
    if (A > 0 && j >= A) {
      int b = 0;
      while (j >= (A << b)) ++b;
      s = (int64_t)base << b;
    }
    if (j % s == 0) {
      if (cnt < cap) pos[cnt] = j;
      ++cnt;
    }
  }
  return cnt;
}

static void check_schedule(void) {
  static const int64_t cases[][3] = {
      {1024, 16, 0}, {1000, 7, 0},     {1, 1, 0},        {0, 4, 0},     {131072, 16, 4096},
      {9000, 16, 4096}, {5000, 16, 512}, {4097, 16, 4096}, {777, 32, 0},  {100, 3, 12},
      {300000, 5, 40}, {262144, 1, 2},  {600000, 16, 4096}};
  const int64_t cap = 400000;
  int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * cap);
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    const int64_t n = cases[i][0], A = cases[i][2];
    const int32_t base = (int32_t)cases[i][1];
    const int64_t cnt = walk_refs(n, base, A, pos, cap);
    CHECK(rkv_num_refs(n, st(base, A)) == cnt);
    for (int64_t s = 0; s < cnt && s < cap; ++s)
      if (rkv_ref_position(s, st(base, A)) != pos[s]) {
        CHECK(rkv_ref_position(s, st(base, A)) == pos[s]);
        break;
      }
  }
  free(pos);
  CHECK(rkv_num_refs(100, st(0, 0)) == -1);
  CHECK(rkv_num_refs(100, st(16, 100)) == -1); /* not a multiple of 2 * base */
  CHECK(rkv_num_refs(-1, st(16, 0)) == -1);
}

static void check_cache_init_and_sizes(void) {
  rkv_cache c = make_cache(2, 8, 8192, 32);
  size_t sz[6];
  const size_t ih = 16, N = 8192;
  CHECK(rkv_cache_init(&c) == RKV_OK);
  CHECK(c.n_refs == 256);
  CHECK(rkv_cache_sizes(&c, sz) == RKV_OK);
  CHECK(sz[0] == ih * N * 8 * 2);
  CHECK(sz[1] == ih * N * 64);
  CHECK(sz[2] == ih * (N / 32) * 128 * 16);
  CHECK(sz[3] == ih * N * 2 * 4 * 2);
  CHECK(sz[4] == ih * 2 * 256 * 128 * 2);
  CHECK(sz[5] == 0);
  c.ref_bits = 4;
  CHECK(rkv_cache_sizes(&c, sz) == RKV_OK);
  CHECK(sz[4] == ih * 2 * 256 * 64 && sz[5] == ih * 2 * 256 * 4 * 2);

  /* rejected descriptions */
  struct {
    int field;
    int64_t value;
    rkv_status want;
  } bad[] = {{0, 0, RKV_ERR_INVALID_ARG},  {0, 17, RKV_ERR_INVALID_ARG},
             {1, 3, RKV_ERR_INVALID_ARG},  {2, 48, RKV_ERR_INVALID_ARG},
             {3, 64, RKV_ERR_UNSUPPORTED}, {4, 0, RKV_ERR_INVALID_ARG},
             {5, 7, RKV_ERR_INVALID_ARG},  {6, 0, RKV_ERR_INVALID_ARG},
             {7, 2, RKV_ERR_RANGE},        {8, 100, RKV_ERR_INVALID_ARG},
             {9, 2, RKV_ERR_INVALID_ARG},  {10, 2, RKV_ERR_INVALID_ARG}};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    rkv_cache b = make_cache(2, 8, 8192, 32);
    switch (bad[i].field) {
      case 0: b.k = (int32_t)bad[i].value; break;
      case 1: b.bits = (int32_t)bad[i].value; break;
      case 2: b.group = (int32_t)bad[i].value; break;
      case 3: b.head_dim = (int32_t)bad[i].value; break;
      case 4: b.stride.base = (int32_t)bad[i].value; break;
      case 5: b.dtype = (rkv_dtype)bad[i].value; break;
      case 6: b.n_kv_heads = (int32_t)bad[i].value; break;
      case 7: b.seq_len = 65536 * 2; b.stride.base = (int32_t)bad[i].value; break;
      case 8: b.stride.base = 16; b.stride.double_after = bad[i].value; break;
      case 9: b.ref_bits = (int32_t)bad[i].value; break;
      case 10: b.latent = (int32_t)bad[i].value; break;
    }
    CHECK(rkv_cache_init(&b) == bad[i].want);
  }
  rkv_cache rb = make_cache(2, 8, 8192, 32);
  rb.ref_bits = 4;
  rb.bits = 0;
  CHECK(rkv_cache_init(&rb) == RKV_ERR_INVALID_ARG);
  rkv_cache lb = make_cache(2, 8, 8192, 32);
  lb.latent = 1;
  lb.bits = 0;
  CHECK(rkv_cache_init(&lb) == RKV_ERR_INVALID_ARG);
  {
    /* the longest sequence the kernels' 32-bit row offsets reach, and one
     * tile more */
    rkv_cache lg = make_cache(1, 1, (int64_t)1 << 22, 1 << 16);
    CHECK(rkv_cache_init(&lg) == RKV_OK && lg.n_refs == 64);
    lg.seq_len += 32;
    CHECK(rkv_cache_init(&lg) == RKV_ERR_INVALID_ARG);
    /* the largest instance and head counts at that length: sizes in range */
    rkv_cache mx = make_cache(65535, 65535, (int64_t)1 << 22, 1 << 16);
    CHECK(rkv_cache_init(&mx) == RKV_OK);
    CHECK(rkv_cache_sizes(&mx, sz) == RKV_OK);
    CHECK(sz[1] == (size_t)65535 * 65535 * ((size_t)1 << 22) * 64);
    CHECK(rkv_decode_split_hint(&mx, 65535, &(int32_t){0}) == RKV_OK);
    {
      /* workspaces at that shape: at least the reference keys and norms
       * (encode) and one fp32 output row per query head (decode) */
      const size_t ih = (size_t)65535 * 65535;
      size_t ws = 0;
      CHECK(rkv_encode_workspace(&mx, &ws) == RKV_OK && ws >= ih * 64 * (256 + 4));
      CHECK(rkv_decode_workspace(&mx, 65535, 1, &ws) == RKV_OK && ws >= ih * 128 * 4);
    }
  }
  CHECK(rkv_cache_init(NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_cache_sizes(NULL, sz) == RKV_ERR_INVALID_ARG);
}

static void check_validation_before_the_device(void) {
  rkv_cache c = make_cache(2, 8, 8192, 32);
  size_t ws = 0;
  const size_t big = (size_t)1 << 40;
  CHECK(rkv_cache_init(&c) == RKV_OK);
  CHECK(rkv_encode(NULL, NULL, &c, NULL, 0, NULL) == RKV_ERR_INVALID_ARG);
  set_buffers(&c, 0x1000);
  CHECK(rkv_select_refs(NULL, NULL, &c, NULL, 0, NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_encode_workspace(&c, &ws) == RKV_OK);
  CHECK(ws >= 16 * 256 * (256 + 4));
  CHECK(rkv_select_refs(P(0x2000), P(0x3000), &c, P(0x4000), ws - 1, NULL) == RKV_ERR_WORKSPACE);
  CHECK(rkv_decode_workspace(&c, 30, 4, &ws) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_workspace(&c, 32, 4, &ws) == RKV_OK);
  CHECK(rkv_decode_attn(P(0x6000), 32, &c, 0.1f, (float *)P(0x5000), 4, P(0x7000), ws - 1, NULL) ==
        RKV_ERR_WORKSPACE);
  {
    const int64_t ranges[][2] = {{-1, 1}, {0, 0}, {8190, 3}, {8192, 1}};
    for (int i = 0; i < 4; ++i)
      CHECK(rkv_append(P(0x2000), P(0x3000), ranges[i][1], &c, ranges[i][0], P(0x4000), big, NULL) ==
            RKV_ERR_INVALID_ARG);
  }
  CHECK(rkv_append(P(0x2000), P(0x3000), 1, &c, 100, P(0x4000), 16, NULL) == RKV_ERR_WORKSPACE);
  CHECK(rkv_decode_attn_len(P(0x6000), 32, &c, 0, 0.1f, (float *)P(0x5000), 4, P(0x7000), ws, NULL) ==
        RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_attn_len(P(0x6000), 32, &c, 8193, 0.1f, (float *)P(0x5000), 4, P(0x7000), ws,
                            NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_attn_tiles(P(0x6000), 32, &c, 0.1f, NULL, 4, (float *)P(0x5000), 4, P(0x7000), ws,
                              NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_attn_tiles(P(0x6000), 32, &c, 0.1f, (const int32_t *)P(0x8000), 0,
                              (float *)P(0x5000), 4, P(0x7000), ws, NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_attn_tiles(P(0x6000), 32, &c, 0.1f, (const int32_t *)P(0x8000), 4,
                              (float *)P(0x5000), 4, P(0x7000), ws - 1, NULL) == RKV_ERR_WORKSPACE);
  c.bits = 0;
  CHECK(rkv_decode_workspace(&c, 32, 4, &ws) == RKV_OK);
  CHECK(rkv_decode_attn(P(0x6000), 32, &c, 0.1f, (float *)P(0x5000), 4, P(0x7000), ws - 1, NULL) ==
        RKV_ERR_WORKSPACE);
  {
    rkv_cache c2 = make_cache(2, 8, 8192, 32); /* n_refs not initialised */
    CHECK(rkv_encode(P(1), P(1), &c2, NULL, 0, NULL) == RKV_ERR_INVALID_ARG);
  }
}

static void check_alignment(void) {
  rkv_cache c = make_cache(2, 8, 8192, 32);
  const size_t big = (size_t)1 << 40;
  const uintptr_t bufs = 0x10000;
  CHECK(rkv_cache_init(&c) == RKV_OK);
  set_buffers(&c, bufs);
  CHECK(rkv_select_refs(P(0x20000), P(0x30000), &c, P(0x40000), 16, NULL) == RKV_ERR_WORKSPACE);
  CHECK(rkv_select_refs(P(0x20008), P(0x30000), &c, P(0x40000), big, NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_quantize(P(0x20000), P(0x30008), &c, P(0x40000), big, NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_select_refs(P(0x20000), P(0x30000), &c, P(0x40008), big, NULL) == RKV_ERR_INVALID_ARG);
  CHECK(rkv_append(P(0x20004), P(0x30000), 1, &c, 5, P(0x40000), big, NULL) == RKV_ERR_INVALID_ARG);
  c.codes_k = (uint8_t *)P(bufs + 8);
  CHECK(rkv_quantize(P(0x20000), P(0x30000), &c, P(0x40000), big, NULL) == RKV_ERR_INVALID_ARG);
  c.codes_k = (uint8_t *)P(bufs);
  c.ref_idx = (uint16_t *)P(bufs + 8);
  CHECK(rkv_quantize(P(0x20000), P(0x30000), &c, P(0x40000), big, NULL) == RKV_ERR_INVALID_ARG);
  c.ref_idx = (uint16_t *)P(bufs);
  CHECK(rkv_decode_attn(P(0x60004), 32, &c, 0.1f, (float *)P(0x50000), 4, P(0x40000), big, NULL) ==
        RKV_ERR_INVALID_ARG);
  CHECK(rkv_decode_attn(P(0x60000), 32, &c, 0.1f, (float *)P(0x50004), 4, P(0x40000), big, NULL) ==
        RKV_ERR_INVALID_ARG);
  CHECK(rkv_reconstruct(&c, (float *)P(0x70002), (float *)P(0x80000), NULL) == RKV_ERR_INVALID_ARG);
}

static void check_split_hint_and_scratch_limit(void) {
  int32_t ns = 0;
  size_t ws = 0;
  rkv_cache layer = make_cache(8, 8, 32768, 64);
  CHECK(rkv_cache_init(&layer) == RKV_OK);
  CHECK(rkv_decode_split_hint(&layer, 32, &ns) == RKV_OK);
  CHECK(ns == 12); /* 256 CUs assumed when no device can be queried */
  rkv_cache step = make_cache(256, 8, 32768, 64);
  CHECK(rkv_cache_init(&step) == RKV_OK);
  CHECK(rkv_decode_split_hint(&step, 32, &ns) == RKV_OK);
  CHECK(ns == 1);
  rkv_cache two = make_cache(1, 2, 100, 16);
  CHECK(rkv_cache_init(&two) == RKV_OK);
  CHECK(rkv_decode_split_hint(&two, 3, &ns) == RKV_ERR_INVALID_ARG);

  CHECK(rkv_decode_workspace(&step, 32, 12, &ws) == RKV_OK);
  CHECK(ws > RKV_SCRATCH_BYTES);
  CHECK(rkv_decode_attn_noalloc(P(0x6000), 32, &step, 0.1f, (float *)P(0x5000), 12, NULL) ==
        RKV_ERR_WORKSPACE);
  CHECK(rkv_decode_workspace(&layer, 32, 12, &ws) == RKV_OK);
  CHECK(ws <= RKV_SCRATCH_BYTES);
  CHECK(rkv_decode_attn_noalloc(P(0x6000), 32, &layer, 0.1f, (float *)P(0x5000), 12, NULL) ==
        RKV_ERR_INVALID_ARG);
}

static void check_layout_limits(void) {
  const size_t big = (size_t)1 << 40;
  rkv_cache c = make_cache(1, 1, 4096, 64);
  CHECK(rkv_cache_init(&c) == RKV_OK);
  set_buffers(&c, 0x10000);
  CHECK(rkv_decode_attn(P(0x6000), 8, &c, 0.1f, (float *)P(0x5000), 2, P(0x7000), big, NULL) ==
        RKV_ERR_UNSUPPORTED);
  c.group = 128;
  CHECK(rkv_decode_attn(P(0x6000), 8, &c, 0.1f, (float *)P(0x5000), 2, P(0x7000), 16, NULL) ==
        RKV_ERR_WORKSPACE);
  rkv_cache many = make_cache(1, 1, 16384, 4);
  CHECK(rkv_cache_init(&many) == RKV_OK);
  CHECK(many.n_refs == 4096);
  set_buffers(&many, 0x10000);
  CHECK(rkv_decode_attn(P(0x6000), 4, &many, 0.1f, (float *)P(0x5000), 2, P(0x7000), big, NULL) ==
        RKV_ERR_UNSUPPORTED);
}

int main(void) {
  check_schedule();
  check_cache_init_and_sizes();
  check_validation_before_the_device();
  check_alignment();
  check_split_hint_and_scratch_limit();
  check_layout_limits();
  for (int s = 0; s < 6; ++s) CHECK(rkv_status_string((rkv_status)s) != NULL);
  CHECK(rkv_version() >= 1);
  if (n_failed) {
    fprintf(stderr, "%d of %d checks failed\n", n_failed, n_checks);
    return 1;
  }
  printf("ok %d\n", n_checks);
  return 0;
}
