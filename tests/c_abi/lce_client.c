/*
 * A plain C client of liblce.so: no PyTorch, only the C ABI of include/lce.h
 * and the HIP runtime for device memory.  Test infrastructure: the GPU test
 * writes seeded inputs to a file, runs this program, and compares what it
 * writes back with the fp64 oracle and with the Python binding.
 *
 *   lce_client IN OUT        fused forward+backward (lce_forward_backward)
 *   lce_client ce IN OUT     standalone in-place cross-entropy (lce_ce_inplace)
 *
 * IN:  int64 N, D, V, chunk_rows, dtype (lce_dtype), reduction, has_bias,
 *      then X [N][D], W [V][D], b [V] (if has_bias) as raw elements of dtype
 *      (4-byte fp32 or 2-byte bf16 / fp16), then int64 targets [N].
 * OUT: float loss [1, or N for LCE_NONE], int64 n_valid, int64 n_bad, then
 *      grad_X [N][D], grad_W [V][D], grad_b [V] (if has_bias) as raw elements.
 * ce IN:  int64 N, V, reduction, then fp32 logits [N][V], int64 targets [N].
 * ce OUT: float loss [1, or N], int64 n_valid, then the fp32 gradient [N][V]
 *         that lce_ce_inplace wrote over the logits.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lce.h"

#define CHECK_HIP(call)                                                        \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));               \
      return 1;                                                                \
    }                                                                          \
  } while (0)

#define CHECK_LCE(call)                                                        \
  do {                                                                         \
    lce_status s_ = (call);                                                    \
    if (s_ != LCE_OK) {                                                        \
      fprintf(stderr, "%s: %s (%s)\n", #call, lce_status_string(s_),           \
              lce_last_error());                                               \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

/* device copy of a host block */
static int upload(void** dev, const void* host, size_t bytes) {
  CHECK_HIP(hipMalloc(dev, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice));
  return 0;
}

static int download(FILE* f, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return 1;
  if (bytes) CHECK_HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  const int bad = bytes && fwrite(host, 1, bytes, f) != bytes;
  free(host);
  return bad;
}

static int run_ce(const char* in_path, const char* out_path) {
  FILE* in = fopen(in_path, "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", in_path);
    return 1;
  }
  int64_t hdr[3];
  if (fread(hdr, sizeof(int64_t), 3, in) != 3) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int64_t N = hdr[0], V = hdr[1];
  const int32_t reduction = (int32_t)hdr[2];
  void* z = read_block(in, (size_t)(N * V) * sizeof(float));
  void* t = read_block(in, (size_t)N * sizeof(int64_t));
  fclose(in);
  if (!z || !t) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  size_t ws_bytes = 0;
  CHECK_LCE(lce_ce_workspace_size(N, V, &ws_bytes));
  const size_t n_loss = reduction == LCE_NONE ? (size_t)N : 1;
  void *dz, *dt, *dloss, *dnv, *ws;
  if (upload(&dz, z, (size_t)(N * V) * sizeof(float)) ||
      upload(&dt, t, (size_t)N * sizeof(int64_t)))
    return 1;
  CHECK_HIP(hipMalloc(&dloss, n_loss * sizeof(float) + 16));
  CHECK_HIP(hipMalloc(&dnv, sizeof(int64_t)));
  CHECK_HIP(hipMalloc(&ws, ws_bytes ? ws_bytes : 256));
  CHECK_LCE(lce_ce_inplace((float*)dz, (const int64_t*)dt, NULL, N, V, -100, reduction, 1.0f,
                           (float*)dloss, (int64_t*)dnv, ws, ws_bytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  FILE* out = fopen(out_path, "wb");
  if (!out) {
    fprintf(stderr, "cannot open %s\n", out_path);
    return 1;
  }
  if (download(out, dloss, n_loss * sizeof(float)) || download(out, dnv, sizeof(int64_t)) ||
      download(out, dz, (size_t)(N * V) * sizeof(float))) {
    fprintf(stderr, "writing %s failed\n", out_path);
    return 1;
  }
  fclose(out);
  hipFree(dz); hipFree(dt); hipFree(dloss); hipFree(dnv); hipFree(ws);
  free(z); free(t);
  printf("lce_client ce: ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "ce") == 0) return run_ce(argv[2], argv[3]);
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT | %s ce IN OUT\n", argv[0], argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int64_t hdr[7];
  if (fread(hdr, sizeof(int64_t), 7, in) != 7) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int64_t N = hdr[0], D = hdr[1], V = hdr[2];
  const size_t es = hdr[4] == LCE_F32 ? 4 : 2;
  const int has_bias = (int)hdr[6];
  void* X = read_block(in, (size_t)(N * D) * es);
  void* W = read_block(in, (size_t)(V * D) * es);
  void* b = has_bias ? read_block(in, (size_t)V * es) : NULL;
  void* t = read_block(in, (size_t)N * sizeof(int64_t));
  fclose(in);
  if (!X || !W || (has_bias && !b) || !t) {
    fprintf(stderr, "short input\n");
    return 1;
  }

  lce_desc d = {0};
  d.N = N;
  d.D = D;
  d.V = V;
  d.ignore_index = -100;
  d.chunk_rows = hdr[3];
  d.dtype = (int32_t)hdr[4];
  d.acc_dtype = LCE_F32;
  d.has_bias = has_bias;
  d.reduction = (int32_t)hdr[5];
  d.acc_policy = LCE_ACCURATE;
  d.flags = LCE_GRAD_X | LCE_GRAD_W | (has_bias ? LCE_GRAD_B : 0u);
  d.chunk_divisor = 1;
  lce_handle* h = NULL;
  CHECK_LCE(lce_create(&d, &h));
  size_t ws_bytes = 0;
  CHECK_LCE(lce_workspace_size(h, &ws_bytes));

  const int none = d.reduction == LCE_NONE;
  const size_t n_loss = none ? (size_t)N : 1;
  void *dX, *dW, *db = NULL, *dt, *dgo = NULL, *dloss, *dgX, *dgW, *dgb = NULL, *dnv, *dnb, *ws;
  if (upload(&dX, X, (size_t)(N * D) * es) || upload(&dW, W, (size_t)(V * D) * es) ||
      (has_bias && upload(&db, b, (size_t)V * es)) ||
      upload(&dt, t, (size_t)N * sizeof(int64_t)))
    return 1;
  if (none) {
    /* the per-row upstream gradient of the 'none' backward: 1 on every row */
    float* ones = (float*)malloc((size_t)(N ? N : 1) * sizeof(float));
    for (int64_t i = 0; i < N; ++i) ones[i] = 1.0f;
    if (upload(&dgo, ones, (size_t)N * sizeof(float))) return 1;
    free(ones);
  }
  CHECK_HIP(hipMalloc(&dloss, n_loss * sizeof(float) + 16));
  CHECK_HIP(hipMalloc(&dgX, (size_t)(N * D) * es + 16));
  CHECK_HIP(hipMalloc(&dgW, (size_t)(V * D) * es + 16));
  if (has_bias) CHECK_HIP(hipMalloc(&dgb, (size_t)V * es + 16));
  CHECK_HIP(hipMalloc(&dnv, sizeof(int64_t)));
  CHECK_HIP(hipMalloc(&dnb, sizeof(int64_t)));
  CHECK_HIP(hipMalloc(&ws, ws_bytes ? ws_bytes : 256));

  lce_io io = {0};
  io.X = dX;
  io.W = dW;
  io.b = db;
  io.targets = (const int64_t*)dt;
  io.grad_output = (const float*)dgo;
  io.loss = (float*)dloss;
  io.grad_X = dgX;
  io.grad_W = dgW;
  io.grad_b = dgb;
  io.argmax = NULL;
  io.n_valid = (int64_t*)dnv;
  io.n_bad = (int64_t*)dnb;
  io.grad_scale = 1.0f;
  io.class_weight = NULL;
  CHECK_LCE(lce_forward_backward(h, &io, ws, ws_bytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    fprintf(stderr, "cannot open %s\n", argv[2]);
    return 1;
  }
  if (download(out, dloss, n_loss * sizeof(float)) || download(out, dnv, sizeof(int64_t)) ||
      download(out, dnb, sizeof(int64_t)) || download(out, dgX, (size_t)(N * D) * es) ||
      download(out, dgW, (size_t)(V * D) * es) ||
      (has_bias && download(out, dgb, (size_t)V * es))) {
    fprintf(stderr, "writing %s failed\n", argv[2]);
    return 1;
  }
  fclose(out);

  CHECK_LCE(lce_destroy(h));
  hipFree(dX); hipFree(dW); hipFree(db); hipFree(dt); hipFree(dgo); hipFree(dloss);
  hipFree(dgX); hipFree(dgW); hipFree(dgb); hipFree(dnv); hipFree(dnb); hipFree(ws);
  free(X); free(W); free(b); free(t);
  printf("lce_client: ok\n");
  return 0;
}
