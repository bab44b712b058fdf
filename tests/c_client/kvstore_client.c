/*
 * A plain C11 client of include/kvstore.h, with no Python and no torch.
 *
 *   kvstore_client validate   argument checks of every entry point (no GPU:
 *                             every call returns before any launch)
 *   kvstore_client gpu        stores through every entry point into hipMalloc'd
 *                             buffers on the current device and compares every
 *                             byte with the CPU oracle (oracle/liboracle.so)
 *   kvstore_client latency    per-call time of decode-size stores issued from C
 *                             (256 tokens of 8 x 128 bf16): back to back, and
 *                             replayed from a captured HIP graph
 *
 * Exit status 0 when every check passed; each failed check prints a line.
 * The oracle is test infrastructure: this program is a test.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvstore.h"

/* The oracle's entry points (oracle/kvstore_oracle.c). */
int64_t oracle_copy(const uint8_t* k, const uint8_t* v, uint8_t* k_cache, uint8_t* v_cache,
                    const void* indices, int idx_is_i64, int64_t idx_stride, int64_t row_bytes,
                    int64_t k_stride, int64_t v_stride, int64_t cache_stride, int64_t batch,
                    int64_t size_limit, int64_t* first_bad, uint64_t* bad_count);
typedef int64_t (*oracle_fp8_fn)(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*,
                                 const void*, int, int64_t, int, int64_t, int64_t, int64_t,
                                 int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                                 int64_t, int64_t, int64_t, int64_t, int64_t, const float*,
                                 const float*, int64_t*, uint64_t*);
int64_t oracle_fp8_paged(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, const void*, int,
                         int64_t, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, const float*, const float*, int64_t*, uint64_t*);
int64_t oracle_fp8_paged_e5m2(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, const void*,
                              int, int64_t, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                              int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                              int64_t, int64_t, int64_t, const float*, const float*, int64_t*,
                              uint64_t*);
int64_t oracle_fp8_paged_dynamic(const uint8_t*, const uint8_t*, uint8_t*, uint8_t*,
                                 const void*, int, int64_t, int, int64_t, int64_t, int64_t,
                                 int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                                 int64_t, int64_t, uint8_t*, uint8_t*, int64_t, int64_t,
                                 int64_t, int64_t, int64_t, int64_t, int, int64_t, int64_t,
                                 int64_t, int64_t*, uint64_t*);

static int g_failures = 0;

#define EXPECT(cond, ...)                              \
  do {                                                 \
    if (!(cond)) {                                     \
      ++g_failures;                                    \
      printf("FAIL %s:%d: ", __FILE__, __LINE__);      \
      printf(__VA_ARGS__);                             \
      printf("\n");                                    \
    }                                                  \
  } while (0)

/* ------------------------------------------------------------------------ */
/* validate: argument checks, no GPU work                                    */
/* ------------------------------------------------------------------------ */

/* Addresses that are never dereferenced: every call below returns before a
 * launch.  A is 256-byte aligned; A + 4 is 4-byte aligned only. */
#define A ((void*)(uintptr_t)0x100000)
#define A4 ((void*)(uintptr_t)0x100004)

static int copy_call(const void* k, void* kc, const void* ix, int idx_dtype, int64_t idx_stride,
                     int64_t row, int64_t ks, int64_t cs, uint32_t batch, int64_t limit) {
  return kvstore_copy(k, k, kc, kc, ix, idx_dtype, idx_stride, row, ks, ks, cs, batch, limit, 0);
}

static int fp8_call(int e5m2, const void* k, void* kc, int idx_dtype, int src, int32_t heads,
                    int32_t dim, int64_t ktok, int64_t khead, int64_t cpage, int64_t coff,
                    int64_t chead, uint32_t batch, int64_t limit, int64_t page,
                    const float* inv) {
  if (e5m2)
    return kvstore_fp8_paged_e5m2(k, k, kc, kc, A, idx_dtype, 1, src, heads, dim, ktok, khead,
                                  ktok, khead, cpage, coff, chead, cpage, coff, chead, batch,
                                  limit, page, inv, inv, 0);
  return kvstore_fp8_paged(k, k, kc, kc, A, idx_dtype, 1, src, heads, dim, ktok, khead, ktok,
                           khead, cpage, coff, chead, cpage, coff, chead, batch, limit, page, inv,
                           inv, 0);
}

static int dyn_call(int gran, int32_t heads, int32_t dim, float* sc, int64_t s_off,
                    int64_t s_head) {
  const int64_t row = (int64_t)heads * dim;
  return kvstore_fp8_paged_dynamic(A, A, A, A, A, KVSTORE_IDX_I32, 1, KVSTORE_SRC_BF16, heads,
                                   dim, 2 * row, 2 * dim, 2 * row, 2 * dim, 64 * row, row, dim,
                                   64 * row, row, dim, sc, sc, gran, 64 * s_off, s_off, s_head,
                                   64 * s_off, s_off, s_head, 10, 640, 64, 0);
}

static void validate(void) {
  const int I32 = KVSTORE_IDX_I32, I64 = KVSTORE_IDX_I64, BF = KVSTORE_SRC_BF16;
  float* sc = (float*)A;

  /* copy */
  EXPECT(copy_call(A, A, A, I32, 1, 2048, 2048, 2048, 0, 10) == KVSTORE_OK, "empty batch");
  EXPECT(copy_call(NULL, NULL, NULL, I32, 1, 2048, 2048, 2048, 0, 10) == KVSTORE_OK,
         "empty batch with NULL pointers");
  EXPECT(copy_call(NULL, A, A, I32, 1, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_NULL, "null k");
  EXPECT(copy_call(A, NULL, A, I32, 1, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_NULL,
         "null cache");
  EXPECT(copy_call(A, A, NULL, I32, 1, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_NULL,
         "null indices");
  EXPECT(copy_call(A, A, A, 2, 1, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_DTYPE,
         "bad index type");
  EXPECT(copy_call(A, A, A, I32, 0, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_SHAPE,
         "index stride 0");
  EXPECT(copy_call(A, A, A, I32, 1, 0, 2048, 2048, 4, 10) == KVSTORE_ERR_SHAPE, "row 0");
  EXPECT(copy_call(A, A, A, I32, 1, 2046, 2048, 2048, 4, 10) == KVSTORE_ERR_SHAPE,
         "row not a multiple of 4");
  EXPECT(copy_call(A, A, A, I32, 1, 2048, 2048, 1024, 4, 10) == KVSTORE_ERR_SHAPE,
         "cache stride below the row");
  EXPECT(copy_call(A, A, A, I32, 1, 2048, 2048, 2048, 4, 0) == KVSTORE_ERR_SHAPE,
         "size limit 0");
  EXPECT(copy_call(A, A, A, I32, 1, 2048, 2048, 2048, 4, INT64_MAX / 1024) == KVSTORE_ERR_SHAPE,
         "cache extent beyond int64");
  EXPECT(copy_call(A, A, A, I32, INT64_MAX / 4, 2048, 2048, 2048, 4, 10) == KVSTORE_ERR_SHAPE,
         "index stride beyond int64 offsets");
  EXPECT(copy_call((const char*)A + 2, A, A, I32, 1, 2048, 2048, 2048, 4, 10) ==
             KVSTORE_ERR_ALIGN,
         "2-byte aligned k");
  EXPECT(copy_call(A, A, (const char*)A + 4, I64, 1, 2048, 2048, 2048, 4, 10) ==
             KVSTORE_ERR_ALIGN,
         "int64 indices 4-byte aligned");
  EXPECT(copy_call(A, A, A, I32, 1, 2048, 2050, 2048, 4, 10) == KVSTORE_ERR_ALIGN,
         "k stride not a multiple of 4");

  /* fp8 (both formats share the checks) */
  for (int e5m2 = 0; e5m2 < 2; ++e5m2) {
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 8, 128, 2048, 256, 65536, 1024, 128, 0, 64, 64, NULL) ==
               KVSTORE_OK,
           "fp8 empty batch (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, NULL, A, I32, BF, 8, 128, 2048, 256, 65536, 1024, 128, 4, 64, 64,
                    NULL) == KVSTORE_ERR_NULL,
           "fp8 null k (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, 2, 8, 128, 2048, 256, 65536, 1024, 128, 4, 64, 64, NULL) ==
               KVSTORE_ERR_DTYPE,
           "fp8 bad source type (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 8, 120, 1920, 240, 61440, 960, 120, 4, 64, 64, NULL) ==
               KVSTORE_ERR_SHAPE,
           "fp8 head_dim not a multiple of 16 (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 0, 128, 2048, 256, 65536, 1024, 128, 4, 64, 64, NULL) ==
               KVSTORE_ERR_SHAPE,
           "fp8 zero heads (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 8, 128, 2048, 256, 65536, 1024, 128, 4, 64, 0, NULL) ==
               KVSTORE_ERR_SHAPE,
           "fp8 page size 0 (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A4, A, I32, BF, 8, 128, 2048, 256, 65536, 1024, 128, 4, 64, 64, NULL) ==
               KVSTORE_ERR_ALIGN,
           "fp8 input 4-byte aligned (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 8, 128, 2048, 256, 65536, 1028, 128, 4, 64, 64, NULL) ==
               KVSTORE_ERR_ALIGN,
           "fp8 slot stride not a multiple of 16 (e5m2=%d)", e5m2);
    EXPECT(fp8_call(e5m2, A, A, I32, BF, 8, 128, 2048, 256, 65536, 1024, 128, 4, 64, 64,
                    (const float*)((const char*)A + 2)) == KVSTORE_ERR_ALIGN,
           "fp8 scale pointer 2-byte aligned (e5m2=%d)", e5m2);
  }

  /* dynamic scales */
  EXPECT(dyn_call(2, 8, 128, sc, 4, 0) == KVSTORE_ERR_DTYPE, "dynamic bad granularity");
  EXPECT(dyn_call(KVSTORE_SCALE_PER_TOKEN, 64, 128, sc, 4, 0) == KVSTORE_ERR_SHAPE,
         "dynamic row beyond 4096 elements");
  EXPECT(dyn_call(KVSTORE_SCALE_PER_TOKEN_HEAD, 4, 80, sc, 16, 4) == KVSTORE_ERR_SHAPE,
         "dynamic per head, head_dim/16 not a power of two");
  EXPECT(dyn_call(KVSTORE_SCALE_PER_TOKEN, 8, 128, NULL, 4, 0) == KVSTORE_ERR_NULL,
         "dynamic null scale cache");
  EXPECT(dyn_call(KVSTORE_SCALE_PER_TOKEN_HEAD, 8, 128, sc, 32, 2) == KVSTORE_ERR_ALIGN,
         "dynamic scale head stride not a multiple of 4");

  /* graph-capturable error take */
  EXPECT(kvstore_take_error(NULL, 0) == KVSTORE_ERR_NULL, "take_error null");
  EXPECT(kvstore_take_error((int64_t*)A4, 0) == KVSTORE_ERR_ALIGN, "take_error misaligned");

  /* status text */
  for (int s = KVSTORE_ERR_OOB; s <= KVSTORE_OK; ++s) {
    const char* t = kvstore_strerror(s);
    EXPECT(t != NULL && t[0] != '\0', "strerror(%d) empty", s);
    for (int r = KVSTORE_ERR_OOB; r < s; ++r)
      EXPECT(t == NULL || strcmp(t, kvstore_strerror(r)) != 0, "strerror(%d) == strerror(%d)",
             s, r);
  }
  EXPECT(kvstore_strerror(12345) != NULL, "strerror of an unknown code");
}

/* ------------------------------------------------------------------------ */
/* gpu: every entry point against the oracle                                 */
/* ------------------------------------------------------------------------ */

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014): seeded input bytes, nothing of the method. */
static uint64_t g_state;
static uint64_t next_u64(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void fill_random(uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)next_u64();
}

/* The first n entries of a random permutation of [0, range), as int32. */
static void random_slots(int32_t* out, int64_t n, int64_t range) {
  int32_t* perm = (int32_t*)malloc((size_t)range * sizeof *perm);
  for (int64_t i = 0; i < range; ++i) perm[i] = (int32_t)i;
  for (int64_t i = range - 1; i > 0; --i) {
    int64_t j = (int64_t)(next_u64() % (uint64_t)(i + 1));
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  memcpy(out, perm, (size_t)n * sizeof *out);
  free(perm);
}

#define HIP_OK(x)                                                            \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

static void* dev_copy_of(const void* host, size_t n) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n));
  HIP_OK(hipMemcpy(d, host, n, hipMemcpyHostToDevice));
  return d;
}

static void* dev_sentinel(size_t n) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n));
  HIP_OK(hipMemset(d, 0xFF, n));
  return d;
}

static void expect_same(const void* dev, const uint8_t* want, size_t n, const char* what) {
  uint8_t* got = (uint8_t*)malloc(n);
  HIP_OK(hipMemcpy(got, dev, n, hipMemcpyDeviceToHost));
  size_t bad = 0, first = 0;
  for (size_t i = 0; i < n; ++i)
    if (got[i] != want[i] && bad++ == 0) first = i;
  EXPECT(bad == 0, "%s: %zu of %zu bytes differ, first at %zu (got 0x%02x want 0x%02x)", what,
         bad, n, first, bad ? got[first] : 0, bad ? want[first] : 0);
  free(got);
}

static void expect_flag(hipStream_t s, int64_t first_bad, uint64_t count, const char* what) {
  int64_t fb = 0;
  uint64_t bc = 0;
  int st = kvstore_check_error(s, &fb, &bc);
  EXPECT(st == (count ? KVSTORE_ERR_OOB : KVSTORE_OK) && fb == first_bad && bc == count,
         "%s: flag (%d, %lld, %llu), oracle (%lld, %llu)", what, st, (long long)fb,
         (unsigned long long)bc, (long long)first_bad, (unsigned long long)count);
}

static void gpu_copy(hipStream_t s) {
  /* 777 tokens of 1040-byte rows (a partial last 1 KiB chunk) read at a
   * 1056-byte stride, into 2048 slots; token 500 carries a bad index. */
  const int64_t T = 777, row = 1040, stride = 1056, slots = 2048;
  uint8_t* k = (uint8_t*)malloc((size_t)(T * stride));
  uint8_t* v = (uint8_t*)malloc((size_t)(T * stride));
  int32_t* ix = (int32_t*)malloc((size_t)T * sizeof *ix);
  fill_random(k, (size_t)(T * stride));
  fill_random(v, (size_t)(T * stride));
  random_slots(ix, T, slots);
  ix[500] = (int32_t)slots;
  void *dk = dev_copy_of(k, (size_t)(T * stride)), *dv = dev_copy_of(v, (size_t)(T * stride));
  void* dix = dev_copy_of(ix, (size_t)T * sizeof *ix);
  const size_t cb = (size_t)(slots * row);
  void *dkc = dev_sentinel(cb), *dvc = dev_sentinel(cb);
  printf("[c-client] copy T=%lld row=%lld\n", (long long)T, (long long)row);
  fflush(stdout);
  int st = kvstore_copy(dk, dv, dkc, dvc, dix, KVSTORE_IDX_I32, 1, row, stride, stride, row,
                        (uint32_t)T, slots, s);
  EXPECT(st == KVSTORE_OK, "kvstore_copy returned %d", st);
  uint8_t *okc = (uint8_t*)malloc(cb), *ovc = (uint8_t*)malloc(cb);
  memset(okc, 0xFF, cb);
  memset(ovc, 0xFF, cb);
  int64_t fb;
  uint64_t bc;
  oracle_copy(k, v, okc, ovc, ix, 0, 1, row, stride, stride, row, T, slots, &fb, &bc);
  expect_flag(s, fb, bc, "copy");
  expect_same(dkc, okc, cb, "copy k_cache");
  expect_same(dvc, ovc, cb, "copy v_cache");
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dix));
  HIP_OK(hipFree(dkc));
  HIP_OK(hipFree(dvc));
  free(k);
  free(v);
  free(ix);
  free(okc);
  free(ovc);
}

/* Static-scale FP8 stores (e4m3fn and e5m2) of random 16-bit patterns: 500
 * tokens of 4 heads x 80 (fp16 then bf16), page size 48, 24 pages. */
static void gpu_fp8(hipStream_t s, int e5m2, int src) {
  const int64_t T = 500, H = 4, D = 80, P = 48, pages = 24, slots = P * pages;
  const int64_t row = H * D, in_bytes = T * row * 2, cb = slots * row;
  uint8_t* k = (uint8_t*)malloc((size_t)in_bytes);
  uint8_t* v = (uint8_t*)malloc((size_t)in_bytes);
  int32_t* ix = (int32_t*)malloc((size_t)T * sizeof *ix);
  fill_random(k, (size_t)in_bytes);
  fill_random(v, (size_t)in_bytes);
  random_slots(ix, T, slots);
  ix[7] = -1;
  const float inv[2] = {0.4f, 1.0f / 1.7f};
  void *dk = dev_copy_of(k, (size_t)in_bytes), *dv = dev_copy_of(v, (size_t)in_bytes);
  void* dix = dev_copy_of(ix, (size_t)T * sizeof *ix);
  float* dinv = (float*)dev_copy_of(inv, sizeof inv);
  void *dkc = dev_sentinel((size_t)cb), *dvc = dev_sentinel((size_t)cb);
  printf("[c-client] fp8 e5m2=%d src=%d T=%lld H=%lld D=%lld P=%lld\n", e5m2, src, (long long)T,
         (long long)H, (long long)D, (long long)P);
  fflush(stdout);
  int st = (e5m2 ? kvstore_fp8_paged_e5m2 : kvstore_fp8_paged)(
      dk, dv, dkc, dvc, dix, KVSTORE_IDX_I32, 1, src, (int32_t)H, (int32_t)D, row * 2, D * 2,
      row * 2, D * 2, P * row, row, D, P * row, row, D, (uint32_t)T, slots, P, dinv, dinv + 1,
      s);
  EXPECT(st == KVSTORE_OK, "fp8 store (e5m2=%d) returned %d", e5m2, st);
  uint8_t *okc = (uint8_t*)malloc((size_t)cb), *ovc = (uint8_t*)malloc((size_t)cb);
  memset(okc, 0xFF, (size_t)cb);
  memset(ovc, 0xFF, (size_t)cb);
  int64_t fb;
  uint64_t bc;
  oracle_fp8_fn ref = e5m2 ? oracle_fp8_paged_e5m2 : oracle_fp8_paged;
  ref(k, v, okc, ovc, ix, 0, 1, src == KVSTORE_SRC_FP16, H, D, row * 2, D * 2, row * 2, D * 2,
      P * row, row, D, P * row, row, D, T, slots, P, &inv[0], &inv[1], &fb, &bc);
  expect_flag(s, fb, bc, "fp8");
  expect_same(dkc, okc, (size_t)cb, e5m2 ? "e5m2 k_cache" : "e4m3fn k_cache");
  expect_same(dvc, ovc, (size_t)cb, e5m2 ? "e5m2 v_cache" : "e4m3fn v_cache");
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dix));
  HIP_OK(hipFree(dinv));
  HIP_OK(hipFree(dkc));
  HIP_OK(hipFree(dvc));
  free(k);
  free(v);
  free(ix);
  free(okc);
  free(ovc);
}

/* Dynamic scales: 300 tokens of 8 heads x 64 bf16, page size 64, 8 pages. */
static void gpu_dynamic(hipStream_t s, int gran) {
  const int64_t T = 300, H = 8, D = 64, P = 64, pages = 8, slots = P * pages;
  const int64_t row = H * D, in_bytes = T * row * 2, cb = slots * row;
  const int64_t G = gran == KVSTORE_SCALE_PER_TOKEN_HEAD ? H : 1, sb = slots * G * 4;
  uint8_t* k = (uint8_t*)malloc((size_t)in_bytes);
  uint8_t* v = (uint8_t*)malloc((size_t)in_bytes);
  int32_t* ix = (int32_t*)malloc((size_t)T * sizeof *ix);
  /* ordinary bf16 magnitudes: random sign and mantissa, exponent 2^-4 .. 2^11 */
  for (int64_t i = 0; i < T * row; ++i) {
    uint64_t r = next_u64();
    uint16_t kb = (uint16_t)((r & 0x807F) | ((123 + (r >> 16) % 16) << 7));
    uint16_t vb = (uint16_t)(((r >> 32) & 0x807F) | ((123 + (r >> 48) % 16) << 7));
    memcpy(k + 2 * i, &kb, 2);
    memcpy(v + 2 * i, &vb, 2);
  }
  random_slots(ix, T, slots);
  ix[T - 1] = (int32_t)slots + 5;
  void *dk = dev_copy_of(k, (size_t)in_bytes), *dv = dev_copy_of(v, (size_t)in_bytes);
  void* dix = dev_copy_of(ix, (size_t)T * sizeof *ix);
  void *dkc = dev_sentinel((size_t)cb), *dvc = dev_sentinel((size_t)cb);
  void *dks = dev_sentinel((size_t)sb), *dvs = dev_sentinel((size_t)sb);
  const int64_t s_head = G > 1 ? 4 : 0;
  printf("[c-client] dynamic granularity=%d T=%lld H=%lld D=%lld\n", gran, (long long)T,
         (long long)H, (long long)D);
  fflush(stdout);
  int st = kvstore_fp8_paged_dynamic(
      dk, dv, dkc, dvc, dix, KVSTORE_IDX_I32, 1, KVSTORE_SRC_BF16, (int32_t)H, (int32_t)D,
      row * 2, D * 2, row * 2, D * 2, P * row, row, D, P * row, row, D, (float*)dks, (float*)dvs,
      gran, P * G * 4, G * 4, s_head, P * G * 4, G * 4, s_head, (uint32_t)T, slots, P, s);
  EXPECT(st == KVSTORE_OK, "dynamic store returned %d", st);
  uint8_t *okc = (uint8_t*)malloc((size_t)cb), *ovc = (uint8_t*)malloc((size_t)cb);
  uint8_t *oks = (uint8_t*)malloc((size_t)sb), *ovs = (uint8_t*)malloc((size_t)sb);
  memset(okc, 0xFF, (size_t)cb);
  memset(ovc, 0xFF, (size_t)cb);
  memset(oks, 0xFF, (size_t)sb);
  memset(ovs, 0xFF, (size_t)sb);
  int64_t fb;
  uint64_t bc;
  oracle_fp8_paged_dynamic(k, v, okc, ovc, ix, 0, 1, 0, H, D, row * 2, D * 2, row * 2, D * 2,
                           P * row, row, D, P * row, row, D, oks, ovs, P * G * 4, G * 4, s_head,
                           P * G * 4, G * 4, s_head, gran == KVSTORE_SCALE_PER_TOKEN_HEAD, T,
                           slots, P, &fb, &bc);
  expect_flag(s, fb, bc, "dynamic");
  expect_same(dkc, okc, (size_t)cb, "dynamic k_cache");
  expect_same(dvc, ovc, (size_t)cb, "dynamic v_cache");
  expect_same(dks, oks, (size_t)sb, "dynamic k_scales");
  expect_same(dvs, ovs, (size_t)sb, "dynamic v_scales");
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dix));
  HIP_OK(hipFree(dkc));
  HIP_OK(hipFree(dvc));
  HIP_OK(hipFree(dks));
  HIP_OK(hipFree(dvs));
  free(k);
  free(v);
  free(ix);
  free(okc);
  free(ovc);
  free(oks);
  free(ovs);
}

static void gpu_take_error(hipStream_t s) {
  /* 64 tokens of 256-byte rows into 128 slots, tokens 40, 3 and 9 out of
   * range: the take reports (3, 3) in device memory and clears the flag. */
  const int64_t T = 64, row = 256, slots = 128;
  uint8_t* k = (uint8_t*)malloc((size_t)(T * row));
  int32_t* ix = (int32_t*)malloc((size_t)T * sizeof *ix);
  fill_random(k, (size_t)(T * row));
  random_slots(ix, T, slots);
  ix[40] = (int32_t)slots;
  ix[3] = (int32_t)(slots + 7);
  ix[9] = -1;
  void* dk = dev_copy_of(k, (size_t)(T * row));
  void* dix = dev_copy_of(ix, (size_t)T * sizeof *ix);
  void *dkc = dev_sentinel((size_t)(slots * row)), *dvc = dev_sentinel((size_t)(slots * row));
  int64_t* dout = (int64_t*)dev_sentinel(2 * sizeof(int64_t));
  printf("[c-client] take_error T=%lld\n", (long long)T);
  fflush(stdout);
  EXPECT(kvstore_copy(dk, dk, dkc, dvc, dix, KVSTORE_IDX_I32, 1, row, row, row, row, (uint32_t)T,
                      slots, s) == KVSTORE_OK, "take_error: store");
  EXPECT(kvstore_take_error(dout, s) == KVSTORE_OK, "take_error: launch");
  HIP_OK(hipStreamSynchronize(s));
  int64_t out[2] = {0, 0};
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  EXPECT(out[0] == 3 && out[1] == 3, "take_error: got (%lld, %lld), want (3, 3)",
         (long long)out[0], (long long)out[1]);
  expect_flag(s, -1, 0, "after take_error");
  EXPECT(kvstore_take_error(dout, s) == KVSTORE_OK, "take_error: second launch");
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  EXPECT(out[0] == -1 && out[1] == 0, "take_error on a clear flag: got (%lld, %lld)",
         (long long)out[0], (long long)out[1]);
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dix));
  HIP_OK(hipFree(dkc));
  HIP_OK(hipFree(dvc));
  HIP_OK(hipFree(dout));
  free(k);
  free(ix);
}

static void gpu(void) {
  g_state = 20240611ull;
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  expect_flag(s, -1, 0, "initial");
  gpu_copy(s);
  gpu_fp8(s, 0, KVSTORE_SRC_FP16);
  gpu_fp8(s, 0, KVSTORE_SRC_BF16);
  gpu_fp8(s, 1, KVSTORE_SRC_BF16);
  gpu_dynamic(s, KVSTORE_SCALE_PER_TOKEN);
  gpu_dynamic(s, KVSTORE_SCALE_PER_TOKEN_HEAD);
  gpu_take_error(s);
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipStreamDestroy(s));
}

/* ------------------------------------------------------------------------ */
/* latency: decode-size calls issued from C                                  */
/* ------------------------------------------------------------------------ */

static double elapsed_us(hipEvent_t a, hipEvent_t b, int calls) {
  float ms = 0.0f;
  HIP_OK(hipEventElapsedTime(&ms, a, b));
  return ms * 1000.0 / calls;
}

static void latency(void) {
  /* 256 tokens of 2 KiB rows, 16 disjoint index sets over 2^20 slots */
  const int64_t T = 256, row = 2048, slots = 1 << 20, H = 8, D = 128, P = 64;
  const int S = 16, N = 2000;
  g_state = 7ull;
  uint8_t* h = (uint8_t*)malloc((size_t)(T * row));
  fill_random(h, (size_t)(T * row));
  void *k = dev_copy_of(h, (size_t)(T * row)), *v = dev_copy_of(h, (size_t)(T * row));
  int32_t* ix = (int32_t*)malloc((size_t)(S * T) * sizeof *ix);
  random_slots(ix, S * T, slots);
  int32_t* dix = (int32_t*)dev_copy_of(ix, (size_t)(S * T) * sizeof *ix);
  void *kc = dev_sentinel((size_t)(slots * row)), *vc = dev_sentinel((size_t)(slots * row));
  const float inv[2] = {0.4f, 1.0f / 1.7f};
  float* dinv = (float*)dev_copy_of(inv, sizeof inv);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  hipEvent_t a, b;
  HIP_OK(hipEventCreate(&a));
  HIP_OK(hipEventCreate(&b));
  for (int op = 0; op < 2; ++op) {
    const char* name = op ? "kvstore_fp8_paged" : "kvstore_copy";
    /* fp8: the same 2 KiB input rows as 8 x 128 bf16, into 1 KiB FP8 slots */
#define CALL(i, st)                                                                          \
  (op ? kvstore_fp8_paged(k, v, kc, vc, dix + ((i) % S) * T, KVSTORE_IDX_I32, 1,               \
                          KVSTORE_SRC_BF16, (int32_t)H, (int32_t)D, row, 2 * D, row, 2 * D,   \
                          P * H * D, H * D, D, P * H * D, H * D, D, (uint32_t)T, slots, P,    \
                          dinv, dinv + 1, st)                                                 \
      : kvstore_copy(k, v, kc, vc, dix + ((i) % S) * T, KVSTORE_IDX_I32, 1, row, row, row,     \
                     row, (uint32_t)T, slots, st))
    for (int i = 0; i < 200; ++i) EXPECT(CALL(i, s) == KVSTORE_OK, "%s warm-up", name);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipEventRecord(a, s));
    for (int i = 0; i < N; ++i) CALL(i, s);
    HIP_OK(hipEventRecord(b, s));
    HIP_OK(hipEventSynchronize(b));
    const double b2b = elapsed_us(a, b, N);
    hipGraph_t g;
    hipGraphExec_t ge;
    HIP_OK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    for (int i = 0; i < S; ++i) CALL(i, s);
    HIP_OK(hipStreamEndCapture(s, &g));
    HIP_OK(hipGraphInstantiate(&ge, g, NULL, NULL, 0));
    for (int r = 0; r < 20; ++r) HIP_OK(hipGraphLaunch(ge, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipEventRecord(a, s));
    for (int r = 0; r < N / S; ++r) HIP_OK(hipGraphLaunch(ge, s));
    HIP_OK(hipEventRecord(b, s));
    HIP_OK(hipEventSynchronize(b));
    const double graph = elapsed_us(a, b, (N / S) * S);
    HIP_OK(hipGraphExecDestroy(ge));
    HIP_OK(hipGraphDestroy(g));
#undef CALL
    printf("[c-client] %s, 256 tokens, from C: %.3f us/call back to back, %.3f us/call "
           "replayed from a graph\n", name, b2b, graph);
  }
  int64_t fb;
  uint64_t bc;
  EXPECT(kvstore_check_error(s, &fb, &bc) == KVSTORE_OK, "latency: flag set");
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(dix));
  HIP_OK(hipFree(kc));
  HIP_OK(hipFree(vc));
  HIP_OK(hipFree(dinv));
  free(h);
  free(ix);
}

int main(int argc, char** argv) {
  if (argc != 2 || (strcmp(argv[1], "validate") != 0 && strcmp(argv[1], "gpu") != 0 &&
                    strcmp(argv[1], "latency") != 0)) {
    fprintf(stderr, "usage: %s validate|gpu|latency\n", argv[0]);
    return 64;
  }
  if (strcmp(argv[1], "validate") == 0)
    validate();
  else if (strcmp(argv[1], "gpu") == 0)
    gpu();
  else
    latency();
  printf("[c-client] %s: %d failure(s)\n", argv[1], g_failures);
  return g_failures ? 1 : 0;
}
