/* Host-side exercise of libarchead under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py builds the
 * library's host code with both and runs this program; no GPU is touched).
 *
 * Every buffer handed to the library is allocated at exactly the size the
 * header documents, so a write or read one byte past it is reported.  Covered:
 * layouts and packing of all three formats over ragged vocabularies, every
 * group size the format allows and zero ranks; the range checks of the codes;
 * the workspace and kernel queries over token counts and paths; the argument
 * checks of every device entry point (each call fails validation before any
 * HIP call, so fake device addresses are never dereferenced).
 * Exit status 0 and one summary line when every expectation held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "archead.h"

static int failures = 0;
#define EXPECT(cond, ...)                        \
  do {                                           \
    if (!(cond)) {                               \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);              \
      fprintf(stderr, "\n");                     \
      ++failures;                                \
    }                                            \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

/* exactly n bytes of random content (n = 0: a one-byte allocation, never read) */
static void* exact(size_t n) {
  unsigned char* p = (unsigned char*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = (unsigned char)rnd();
  return p;
}
static int8_t* codes(size_t n, int lo, int hi) {
  int8_t* p = (int8_t*)exact(n);
  for (size_t i = 0; i < n; ++i) p[i] = (int8_t)(lo + (int)(rnd() % (uint32_t)(hi - lo + 1)));
  return p;
}
static uint16_t* halves(size_t n) { /* finite fp16 bit patterns */
  uint16_t* p = (uint16_t*)exact(2 * n);
  for (size_t i = 0; i < n; ++i) p[i] = (uint16_t)(rnd() % 0x7c00u);
  return p;
}

static void pack_case(int64_t V, int64_t D, int r_c, int r_r, int g, int fmt) {
  archead_dims d = {V, D, r_c, r_r, g, fmt};
  archead_layout L;
  int rc = archead_pack_layout(&d, &L);
  EXPECT(rc == ARCHEAD_OK, "layout V=%lld D=%lld fmt=%d: %d", (long long)V, (long long)D, fmt, rc);
  if (rc) return;
  const int64_t ng = D / g;
  archead_host_components c;
  memset(&c, 0, sizeof c);
  void* keep[16];
  int nk = 0;
  if (fmt == ARCHEAD_FMT_ARCHEAD) {
    keep[nk++] = (void*)(c.q4 = codes((size_t)(V * D), -8, 7));
    keep[nk++] = (void*)(c.c8 = (const uint8_t*)exact((size_t)(V * ng)));
    keep[nk++] = (void*)(c.s_R = halves((size_t)V));
    if (r_c) {
      keep[nk++] = (void*)(c.A_c = codes((size_t)(V * r_c), -127, 127));
      keep[nk++] = (void*)(c.s_Ac = halves((size_t)V));
      keep[nk++] = (void*)(c.B_c = codes((size_t)(r_c * D), -127, 127));
      keep[nk++] = (void*)(c.s_Bc = halves((size_t)(r_c * ng)));
    }
    if (r_r) {
      keep[nk++] = (void*)(c.A_w = codes((size_t)(V * r_r), -127, 127));
      keep[nk++] = (void*)(c.s_Aw = halves((size_t)V));
      keep[nk++] = (void*)(c.B_w = codes((size_t)(r_r * D), -127, 127));
      keep[nk++] = (void*)(c.s_Bw = halves((size_t)(r_r * ng)));
    }
  } else if (fmt == ARCHEAD_FMT_GROUP_INT4) {
    keep[nk++] = (void*)(c.q4 = codes((size_t)(V * D), -8, 7));
    keep[nk++] = (void*)(c.s_G = halves((size_t)(V * ng)));
  } else {
    keep[nk++] = (void*)(c.q8 = codes((size_t)(V * D), -127, 127));
    keep[nk++] = (void*)(c.s_R = halves((size_t)V));
  }
  unsigned char* dst = (unsigned char*)malloc(L.total_bytes);
  rc = archead_pack(&d, &c, dst, L.total_bytes);
  EXPECT(rc == ARCHEAD_OK, "pack V=%lld D=%lld r=%d+%d g=%d fmt=%d: %d", (long long)V, (long long)D, r_c, r_r, g,
         fmt, rc);
  uint32_t flags;
  memcpy(&flags, dst + 36, 4);
  EXPECT(flags == (uint32_t)fmt, "flags %u", flags);
  EXPECT(archead_pack(&d, &c, dst, L.total_bytes - 1) == ARCHEAD_E_SIZE, "short buffer");
  /* one code out of range: nothing written, E_VALUE */
  int8_t* q = (int8_t*)(fmt == ARCHEAD_FMT_ROW_INT8 ? c.q8 : c.q4);
  const size_t at = (size_t)(rnd() % (uint32_t)(V * D));
  const int8_t save = q[at];
  q[at] = fmt == ARCHEAD_FMT_ROW_INT8 ? (int8_t)-128 : (int8_t)8;
  memset(dst, 0xab, L.total_bytes);
  EXPECT(archead_pack(&d, &c, dst, L.total_bytes) == ARCHEAD_E_VALUE, "bad code");
  EXPECT(dst[0] == 0xab && dst[L.total_bytes - 1] == 0xab, "wrote on failure");
  q[at] = save;
  free(dst);
  for (int i = 0; i < nk; ++i) free(keep[i]);
}

static void query_case(int64_t V, int64_t D, int r_c, int r_r, int g, int fmt) {
  archead_dims d = {V, D, r_c, r_r, g, fmt};
  const int64_t ns[] = {0, 1, 2, 4, 5, 16, 17, 31, 32, 33, 63, 64, 65, 256, 257, 1100, 4096};
  for (size_t i = 0; i < sizeof ns / sizeof ns[0]; ++i) {
    for (int path = -1; path <= 3; ++path) {
      uint64_t b = 0;
      int k = -1;
      const int rw = archead_workspace_bytes_path(&d, ns[i], path, &b);
      const int rk = archead_main_kernel(&d, ns[i], path, &k);
      EXPECT(rw == ARCHEAD_OK || rw == ARCHEAD_E_UNSUPPORTED, "workspace rc %d", rw);
      EXPECT(rk == ARCHEAD_OK || rk == ARCHEAD_E_UNSUPPORTED, "main kernel rc %d", rk);
      if (path < 0 || path > 2) EXPECT(rw == ARCHEAD_E_UNSUPPORTED && rk == ARCHEAD_E_UNSUPPORTED, "bad path");
      if (rk == ARCHEAD_OK) EXPECT(k >= 0 && k <= 3, "kernel %d", k);
    }
    uint64_t b = 0;
    (void)archead_workspace_bytes(&d, ns[i], &b);
    (void)archead_stats_workspace_bytes(&d, ns[i], &b);
    (void)archead_topk_workspace_bytes(&d, ns[i], &b);
    (void)archead_logit_error_workspace_bytes(&d, ns[i], &b);
  }
  uint64_t b = 0;
  (void)archead_fit_workspace_bytes(&d, 8, &b);
}

/* Device entry points with arguments that fail validation (fake addresses) */
static void device_errors(void) {
  void* fake = (void*)(uintptr_t)(1ull << 40);
  archead_dims d = {1024, 256, 16, 8, 64, 0};
  archead_tensor H = {fake, 4, 256, 256, ARCHEAD_BF16};
  archead_tensor Y = {fake, 4, 1024, 1024, ARCHEAD_F32};
  archead_packed_head P = {d, fake, 1 << 20, fake, 1 << 20};
  EXPECT(archead_logits(NULL, &P, &Y, NULL) == ARCHEAD_E_NULL, "null H");
  H.dtype = ARCHEAD_F32;
  EXPECT(archead_logits(&H, &P, &Y, NULL) == ARCHEAD_E_DTYPE, "H dtype");
  H.dtype = ARCHEAD_BF16;
  Y.cols = 1000;
  EXPECT(archead_logits(&H, &P, &Y, NULL) == ARCHEAD_E_SHAPE, "Y cols");
  Y.cols = 1024;
  P.buffer = (void*)((uintptr_t)fake + 16);
  EXPECT(archead_logits(&H, &P, &Y, NULL) == ARCHEAD_E_ALIGN, "buffer align");
  P.buffer = fake;
  P.buffer_bytes = 100;
  EXPECT(archead_logits(&H, &P, &Y, NULL) == ARCHEAD_E_SIZE, "buffer size");
  P.buffer_bytes = 1 << 20;
  EXPECT(archead_logits_path(&H, &P, &Y, 7, NULL) == ARCHEAD_E_UNSUPPORTED, "path");
  P.dims.format = 3;
  EXPECT(archead_logits(&H, &P, &Y, NULL) == ARCHEAD_E_DIMS, "format");
  P.dims.format = 1;
  EXPECT(archead_logits_noalloc(&H, &P, &Y, NULL) == ARCHEAD_E_DIMS, "noalloc: factors on a comparison head");
  P.dims = d;
  archead_row_stats st = {fake, fake, fake, fake, NULL};
  EXPECT(archead_logits_stats(&H, &P, &st, NULL) == ARCHEAD_E_NULL, "ce without targets");
  float* tv = (float*)fake;
  int32_t* ti = (int32_t*)fake;
  EXPECT(archead_logits_topk(&H, &P, 0, tv, ti, NULL) == ARCHEAD_E_SHAPE, "k = 0");
  EXPECT(archead_logits_topk(&H, &P, 17, tv, ti, NULL) == ARCHEAD_E_UNSUPPORTED, "k = 17");
  double sums[2];
  archead_tensor W = {fake, 1000, 256, 256, ARCHEAD_BF16};
  EXPECT(archead_logit_error(&H, &P, &W, sums, NULL) == ARCHEAD_E_SHAPE, "W rows");
  archead_dense_head dense;
  memset(&dense, 0, sizeof dense);
  dense.W = fake;
  dense.W_stride = 256;
  dense.W_dtype = ARCHEAD_BF16;
  EXPECT(archead_quantize(&d, &dense, fake, 1 << 30, NULL, NULL) == ARCHEAD_E_NULL, "quantize without factors");
  for (int s = -1; s <= 12; ++s) EXPECT(archead_status_string(s) != NULL, "status string");
}

int main(void) {
  const int64_t Vs[] = {1, 15, 16, 17, 37, 129};
  const int64_t Ds[] = {128, 256, 384, 512};
  const int gs[] = {2, 32, 64, 128, 256};
  const int ranks[][2] = {{0, 0}, {8, 0}, {0, 24}, {16, 8}, {6, 2}};
  int cases = 0;
  for (size_t a = 0; a < sizeof Vs / sizeof Vs[0]; ++a)
    for (size_t b = 0; b < sizeof Ds / sizeof Ds[0]; ++b)
      for (size_t c = 0; c < sizeof gs / sizeof gs[0]; ++c) {
        if (Ds[b] % gs[c]) continue;
        for (size_t r = 0; r < sizeof ranks / sizeof ranks[0]; ++r, ++cases) {
          pack_case(Vs[a], Ds[b], ranks[r][0], ranks[r][1], gs[c], ARCHEAD_FMT_ARCHEAD);
          query_case(Vs[a], Ds[b], ranks[r][0], ranks[r][1], gs[c], ARCHEAD_FMT_ARCHEAD);
        }
        for (int fmt = 1; fmt <= 2; ++fmt, ++cases) {
          pack_case(Vs[a], Ds[b], 0, 0, gs[c], fmt);
          query_case(Vs[a], Ds[b], 0, 0, gs[c], fmt);
        }
      }
  /* full-size shapes: queries only */
  query_case(151936, 4096, 32, 32, 128, 0);
  query_case(151936, 4096, 64, 64, 128, 0);
  query_case(128256, 8192, 64, 64, 128, 0);
  query_case(151936, 8192, 0, 0, 32, 1);
  query_case(151936, 4096, 0, 0, 128, 2);
  query_case((int64_t)1 << 33, 4096, 32, 32, 128, 0);
  device_errors();
  printf("sanitize driver: %d pack/query cases, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
