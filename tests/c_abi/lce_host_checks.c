/*
 * Host-side checks of liblce's planner and validation, for a build of the C
 * ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no
 * GPU needed, no kernel is launched).  Test infrastructure.
 *
 * It walks a grid of valid and invalid problem descriptions (sizes around
 * every limit, each dtype, policy, reduction, flag set, chunk and group size)
 * plus seeded random ones, and for each created handle queries the workspace
 * size and the chunk plan and checks their basic invariants.  It then drives
 * every host-side error path of lce_forward_backward, lce_ce_inplace,
 * lce_ce_inplace_noalloc and lce_scale with pointers that are never
 * dereferenced, because validation fails first.  The sanitizers report any
 * out-of-bounds access, overflow or undefined shift in that code.
 * Prints "ok <handles created> <descriptions tried>" and exits 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lce.h"

static int failures = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

/* splitmix64: a fixed, seeded stream of test descriptions */
static uint64_t rng_state = 0x1234567u;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int64_t pick(const int64_t* v, int n) { return v[next_u64() % (uint64_t)n]; }

static long created = 0, tried = 0;

static void check_desc(const lce_desc* d) {
  lce_handle* h = NULL;
  ++tried;
  const lce_status st = lce_create(d, &h);
  if (st != LCE_OK) {
    EXPECT(h == NULL);
    EXPECT(st == LCE_ERR_INVALID_ARG || st == LCE_ERR_DTYPE || st == LCE_ERR_UNSUPPORTED);
    return;
  }
  ++created;
  size_t ws = 0;
  int64_t c = -1, k = -1;
  EXPECT(lce_workspace_size(h, &ws) == LCE_OK);
  EXPECT(lce_chunk_info(h, &c, &k) == LCE_OK);
  EXPECT(lce_chunk_info(h, NULL, NULL) == LCE_OK);
  if (d->N == 0) {
    EXPECT(c == 0 && k == 0);
  } else {
    EXPECT(c >= 1 && c <= d->N);
    EXPECT(k >= 1 && (k - 1) * c < d->N && k * c >= d->N);
  }
  /* every plan holds at least the per-row arrays and the counters */
  EXPECT(ws >= 24);
  if (d->N > 0 && (d->flags & (LCE_GRAD_X | LCE_GRAD_W | LCE_GRAD_B))) {
    /* the exp / dL tile of one chunk: c rows x V classes of the element type */
    const size_t es = d->dtype == LCE_F32 ? 4 : 2;
    EXPECT(ws / es / (size_t)d->V >= (size_t)c);
  }
  /* host validation of a call: each of these fails before anything is
     enqueued, so the pointers (never dereferenced) need not be real */
  void* fake = (void*)(uintptr_t)(1u << 20);
  lce_io io;
  memset(&io, 0, sizeof io);
  io.X = fake; io.W = fake; io.targets = (const int64_t*)fake; io.loss = (float*)fake;
  io.grad_X = fake; io.grad_W = fake; io.grad_b = fake; io.argmax = (int32_t*)fake;
  io.b = d->has_bias ? fake : NULL;
  io.grad_scale = 1.0f;
  if (ws > 0) {
    EXPECT(lce_forward_backward(h, &io, NULL, ws, NULL) == LCE_ERR_WORKSPACE);
    EXPECT(lce_forward_backward(h, &io, fake, ws - 1, NULL) == LCE_ERR_WORKSPACE);
    EXPECT(lce_forward_backward(h, &io, (char*)fake + 16, ws, NULL) == LCE_ERR_WORKSPACE);
  }
  EXPECT(lce_forward_backward(h, NULL, fake, ws, NULL) == LCE_ERR_INVALID_ARG);
  io.b = d->has_bias ? NULL : fake;
  EXPECT(lce_forward_backward(h, &io, fake, ws, NULL) == LCE_ERR_INVALID_ARG);
  io.b = d->has_bias ? fake : NULL;
  if (d->reduction != LCE_NONE) {
    io.grad_output = (const float*)fake;
    EXPECT(lce_forward_backward(h, &io, fake, ws, NULL) == LCE_ERR_INVALID_ARG);
    io.grad_output = NULL;
    io.loss = NULL;
    EXPECT(lce_forward_backward(h, &io, fake, ws, NULL) == LCE_ERR_INVALID_ARG);
    io.loss = (float*)fake;
  }
  if (d->N > 0) {
    io.X = (char*)fake + 2;                     /* misaligned rows */
    EXPECT(lce_forward_backward(h, &io, fake, ws, NULL) == LCE_ERR_UNSUPPORTED);
    io.X = fake;
    io.targets = NULL;
    EXPECT(lce_forward_backward(h, &io, fake, ws, NULL) == LCE_ERR_INVALID_ARG);
  }
  EXPECT(lce_destroy(h) == LCE_OK);
}

int main(void) {
  const int64_t Ns[] = {0, 1, 3, 64, 300, 1000, 8192, 16384, 1 << 20, (1 << 21) + 5,
                        2147483647LL - 1024, 2147483647LL, -1};
  const int64_t Ds[] = {1, 4, 8, 60, 64, 520, 4096, 1 << 20, (1 << 20) + 8, -8, 0};
  const int64_t Vs[] = {1, 2, 7, 255, 257, 1000, 32000, 128256, 151936, (1 << 21) - 256,
                        (1 << 21) - 255, 1 << 22, 0, -3};
  const int64_t Cs[] = {LCE_CHUNK_ALL, LCE_CHUNK_ASPECT_RATIO, 1, 3, 64, 300, 2048,
                        1 << 20, (1 << 20) + 1, -2};
  const int64_t Gs[] = {0, 1, 64, 2048, 4096, 8192, 1 << 30, -1};
  const int64_t dtypes[] = {LCE_F32, LCE_BF16, LCE_F16, 3, -1};
  const int64_t reds[] = {LCE_MEAN, LCE_SUM, LCE_NONE, 3, -1};
  const int64_t pols[] = {LCE_ACCURATE, LCE_COMPACT, 2};
  const int64_t flag_sets[] = {0, LCE_GRAD_X, LCE_GRAD_W, LCE_GRAD_B,
                               LCE_GRAD_X | LCE_GRAD_W, LCE_GRAD_X | LCE_GRAD_W | LCE_GRAD_B,
                               LCE_GRAD_X | LCE_GRAD_W | LCE_ARGMAX | LCE_ACCUMULATE, 32};
  /* the named workloads, each dtype, policy and group size */
  const int64_t shapes[][4] = {{256, 64, 1000, 64}, {4096, 2048, 32000, 1024},
                               {8192, 4096, 128256, 2048}, {16384, 4096, 151936, 0},
                               {1100, 520, 3001, 300}};
  for (int s = 0; s < 5; ++s)
    for (int dt = 0; dt < 3; ++dt)
      for (int p = 0; p < 2; ++p)
        for (int g = 0; g < 8; ++g)
          for (int r = 0; r < 3; ++r) {
            lce_desc d;
            memset(&d, 0, sizeof d);
            d.N = shapes[s][0]; d.D = shapes[s][1]; d.V = shapes[s][2];
            d.chunk_rows = shapes[s][3]; d.ignore_index = -100;
            d.dtype = (int32_t)dtypes[dt]; d.acc_dtype = LCE_F32; d.has_bias = 1;
            d.reduction = (int32_t)reds[r]; d.acc_policy = (int32_t)pols[p];
            d.flags = LCE_GRAD_X | LCE_GRAD_W | LCE_GRAD_B | LCE_ARGMAX;
            d.group_rows = Gs[g];
            check_desc(&d);
            d.acc_dtype = d.dtype;           /* the non-mixed layout */
            check_desc(&d);
          }
  /* seeded random descriptions around every limit */
  for (int i = 0; i < 40000; ++i) {
    lce_desc d;
    memset(&d, 0, sizeof d);
    d.N = pick(Ns, sizeof Ns / sizeof Ns[0]);
    d.D = pick(Ds, sizeof Ds / sizeof Ds[0]);
    d.V = pick(Vs, sizeof Vs / sizeof Vs[0]);
    d.chunk_rows = pick(Cs, sizeof Cs / sizeof Cs[0]);
    d.group_rows = pick(Gs, sizeof Gs / sizeof Gs[0]);
    d.dtype = (int32_t)pick(dtypes, 5);
    d.acc_dtype = (next_u64() & 1) ? LCE_F32 : (int32_t)pick(dtypes, 5);
    d.reduction = (int32_t)pick(reds, 5);
    d.acc_policy = (int32_t)pick(pols, 3);
    d.has_bias = (int32_t)(next_u64() % 3);
    d.flags = (uint32_t)pick(flag_sets, 8);
    d.chunk_divisor = (int64_t)(next_u64() % 5) - 1;
    d.ignore_index = (next_u64() & 1) ? -100 : 7;
    check_desc(&d);
  }
  EXPECT(lce_create(NULL, NULL) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_destroy(NULL) == LCE_OK);
  EXPECT(lce_workspace_size(NULL, NULL) == LCE_ERR_INVALID_ARG);
  for (int s = -1; s < 8; ++s) EXPECT(lce_status_string((lce_status)s) != NULL);
  EXPECT(lce_last_error() != NULL);

  /* standalone CE: workspace sizes and host validation */
  void* fake = (void*)(uintptr_t)(1u << 20);
  size_t ws = 0;
  EXPECT(lce_ce_workspace_size(16384, 131072, &ws) == LCE_OK && ws >= 4 * 16384 * 4);
  EXPECT(lce_ce_workspace_size(0, 1, &ws) == LCE_OK && ws > 0);
  EXPECT(lce_ce_workspace_size(-1, 1, &ws) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_ce_workspace_size(1, 1, NULL) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_ce_inplace((float*)((char*)fake + 2), (const int64_t*)fake, NULL, 16, 1022, -100,
                        LCE_MEAN, 1.0f, (float*)fake, NULL, fake, 1 << 20, NULL) ==
         LCE_ERR_UNSUPPORTED);                        /* logits not 4-byte aligned */
  EXPECT(lce_ce_inplace((float*)fake, (const int64_t*)fake, NULL, 16, 1024, -100, 3, 1.0f,
                        (float*)fake, NULL, fake, 1 << 20, NULL) == LCE_ERR_UNSUPPORTED);
  EXPECT(lce_ce_inplace((float*)fake, (const int64_t*)fake, NULL, 16, 1024, -100, LCE_MEAN, 1.0f,
                        (float*)fake, NULL, fake, 16, NULL) == LCE_ERR_WORKSPACE);
  EXPECT(lce_ce_inplace(NULL, (const int64_t*)fake, NULL, 16, 1024, -100, LCE_MEAN, 1.0f,
                        (float*)fake, NULL, fake, 1 << 20, NULL) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_ce_inplace_noalloc((float*)fake, (const int64_t*)fake, NULL,
                                LCE_CE_NOALLOC_MAX_ROWS + 1, 1024, -100, LCE_MEAN, 1.0f,
                                (float*)fake, NULL, NULL) == LCE_ERR_UNSUPPORTED);
  EXPECT(strstr(lce_last_error(), "static scratch") != NULL);
  EXPECT(lce_ce_inplace_noalloc((float*)fake, (const int64_t*)fake, NULL, 16, 1024, -100, 5,
                                1.0f, (float*)fake, NULL, NULL) == LCE_ERR_UNSUPPORTED);
  /* lce_scale: every host error */
  const float one = 1.0f;
  EXPECT(lce_scale(fake, fake, LCE_BF16, -1, 8, &one, 0, NULL) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_scale(fake, fake, 9, 1, 8, &one, 0, NULL) == LCE_ERR_DTYPE);
  EXPECT(lce_scale(fake, fake, LCE_BF16, 0, 8, &one, 0, NULL) == LCE_OK);   /* no work */
  EXPECT(lce_scale(NULL, fake, LCE_BF16, 1, 8, &one, 0, NULL) == LCE_ERR_INVALID_ARG);
  EXPECT(lce_scale((char*)fake + 2, fake, LCE_BF16, 1, 8, &one, 0, NULL) == LCE_ERR_UNSUPPORTED);
  EXPECT(lce_scale(fake, fake, LCE_BF16, 1, 6, &one, 1, NULL) == LCE_ERR_UNSUPPORTED);
  EXPECT(lce_scale(fake, fake, LCE_F32, INT64_MAX / 2, 4, &one, 0, NULL) == LCE_ERR_INVALID_ARG);
  if (failures) {
    fprintf(stderr, "%d failed checks\n", failures);
    return 1;
  }
  printf("ok %ld %ld\n", created, tried);
  return 0;
}
