/*
 * lce.h -- C ABI of the chunked fused linear-cross-entropy library (liblce.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For inputs X[N,D], an output-head weight W[V,D], an
 * optional bias b[V] and int64 targets t[N], the logits are z = X W^T + b.
 * The library forms the row-wise log-sum-exp, the per-row loss
 * lse_n - z[n, t_n] (0 on ignored rows), its mean / sum / per-row value, and
 * the gradients grad_X = dL W, grad_W = dL^T X and grad_b = sum_n dL[n, :],
 * where dL = g (softmax(z) - onehot(t)) and g is the per-row weight of the
 * reduction.  It walks the batch rows in chunks of chunk_rows rows and forms
 * the gradients during the same pass as the loss.  The fp32 logits of a chunk
 * exist only in registers, one 256 x 256 output tile at a time, and are never
 * written to memory; what a chunk leaves in the workspace is a tile of
 * (chunk rows x V) in the input dtype:
 *   - bf16 gradients: exp(z - r_n) with one reference r_n per row, its
 *     target logit, and S_n = sum_v exp(z - r_n) taken off the target entry.
 *     That is dL up to the row factor g_n / S_n, which the gradient products
 *     apply (grad_X's rows as they are stored, X's rows as they are staged
 *     for grad_W, the rows of the grad_b sums), so no pass rewrites the
 *     tile.  A row whose largest logit exceeds r_n by more than 40 (a loss
 *     above 40 nats, where exp(z - r_n) could overflow) has the 256-row
 *     tile that holds it recomputed, on the device, with the row max as its
 *     reference.
 *   - fp16 and fp32 (and bf16 with the staged dL^T below): exp(z - block
 *     max), rewritten in place into dL by a finalize pass.
 * Which rows of that tile the workspace holds at once depends on the grad_W
 * accumulation (lce_acc_policy, lce_desc.group_rows):
 *   - ACCURATE with group_rows = 0 (the default) keeps the dL of a group of
 *     consecutive chunks, up to 4 D / sizeof(element) rows (as many bytes as
 *     an fp32 V x D accumulator), and runs one grad_X and one grad_W GEMM
 *     over the whole group.  When that covers every row (e.g. N = 8192,
 *     D = 4096, bf16: one group of N rows, 2.1 GB of bf16 dL), no fp32
 *     accumulator is needed and grad_W is rounded once from fp32 registers.
 *   - ACCURATE with group_rows <= chunk rows keeps one chunk's dL: both
 *     gradient GEMMs consume it as soon as it is complete, and grad_W is
 *     carried across chunks in an fp32 V x D accumulator in the workspace,
 *     rounded once after the last chunk.
 *   - COMPACT keeps one chunk's dL and adds each chunk's grad_W into the
 *     16-bit output (no V x D accumulator).
 *
 * Sources: the PyTorch module source torch/nn/modules/linear_cross_entropy.py
 * (custom ops _linear_cross_entropy_batch_chunked and
 * _linear_cross_entropy_batch_chunked_no_reduction, their argument lists and
 * fake-tensor output contract; _ChunkContext.build validation;
 * neg_weight_target for the per-row weights), the
 * torch.nn.LinearCrossEntropyOptions documentation page (batch_chunk_size,
 * chunking_method "aspect_ratio", acc_policy, acc_dtype), and Liger-Kernel
 * issue #343 (a cross-entropy kernel that overwrites its logits with the
 * gradient in place).
 *
 * Conventions for every entry point:
 *   - Device pointers live on the current HIP device (hipSetDevice /
 *     torch.cuda.set_device); the library never changes the device.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Compute entry points only enqueue work on it: no host synchronisation,
 *     no device allocation.  Errors found on the host are returned before
 *     anything is enqueued.
 *   - The caller owns every device buffer, including the workspace; the
 *     library owns only the host-side handle.  Inputs are never modified,
 *     except the logits buffer of lce_ce_inplace and
 *     lce_ce_inplace_noalloc, which by contract is overwritten with the
 *     gradient.
 *   - All matrices are dense row-major with the row length as stride.
 *   - bf16 tensors are raw bfloat16 bit patterns, fp16 tensors IEEE binary16
 *     (both uint16_t in memory).
 *   - Rows of X and W must be 16-byte aligned: D % 8 == 0 for bf16 / fp16,
 *     D % 4 == 0 for fp32 (LCE_ERR_UNSUPPORTED otherwise); base pointers
 *     16-byte aligned.  The standalone CE takes any V and logits aligned
 *     to 4 bytes.
 *   - Size limits of lce_create (LCE_ERR_UNSUPPORTED otherwise): N, V and D
 *     below 2^31 - 1024; D <= 2^20 and rows per chunk <= 2^20; fp32 inputs
 *     that request grad_X also need V <= 2^21 - 256.  (The GEMMs address a
 *     256-row operand tile with 32-bit offsets.)
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define LCE_API __attribute__((visibility("default")))
#else
#define LCE_API
#endif

typedef struct lce_handle lce_handle;  /* opaque, host memory only */

/* Status codes.  Host validation maps the pages' Python exceptions
 * (_ChunkContext.build: TypeError / NotImplementedError / RuntimeError for
 * bad dtypes, unsupported reductions, shape mismatches) onto these. */
typedef enum {
  LCE_OK = 0,
  LCE_ERR_INVALID_ARG = 1,  /* negative size, NULL required pointer, bad enum */
  LCE_ERR_DTYPE = 2,        /* dtype not in {LCE_F32, LCE_BF16, LCE_F16} */
  LCE_ERR_UNSUPPORTED = 3,  /* unsupported acc_dtype, unaligned rows, ... */
  LCE_ERR_WORKSPACE = 4,    /* workspace NULL, misaligned or too small */
  LCE_ERR_HIP = 5           /* a HIP launch or runtime call failed */
} lce_status;

/* Element types.  bf16 and fp16 accumulate in fp32 (the pages' mixed
 * precision with acc_dtype float32); fp16 keeps the logits gradient scaled by
 * a power of two inside the library so that it stays in fp16's range.
 *
 * acc_dtype (torch.nn.LinearCrossEntropyOptions page: acc_dtype; the module
 * source's dtype layout) is LCE_F32, or the input dtype itself.  For bf16 /
 * fp16 inputs the latter is the non-mixed layout: the gradients accumulate
 * chunk by chunk in the input dtype (grad_W rounded into the 16-bit output
 * after every chunk, as LCE_COMPACT does, whatever acc_policy says).  The
 * logits and softmax statistics are still formed in fp32 on chip; the matrix
 * cores accumulate in fp32 for every input type. */
typedef enum { LCE_F32 = 0, LCE_BF16 = 1, LCE_F16 = 2 } lce_dtype;

/* Loss reduction (the pages' reduction argument). */
typedef enum { LCE_MEAN = 0, LCE_SUM = 1, LCE_NONE = 2 } lce_reduction;

/* How grad_W is accumulated across chunks when the input dtype is bf16 or
 * fp16 (torch.nn.LinearCrossEntropyOptions page: acc_policy "accurate" /
 * "compact").  ACCURATE accumulates grad_W in fp32 over every row and rounds
 * it once: within a group of chunks in the GEMM's fp32 registers, across
 * groups in an fp32 V x D accumulator in the workspace (see the file comment
 * and lce_desc.group_rows for how many chunks form a group).  COMPACT adds
 * each chunk's fp32 product straight into the 16-bit grad_W (one rounding
 * per chunk, at the size of what grad_W then holds, including values that
 * LCE_ACCUMULATE adds to) and needs no V x D accumulator.  Identical for
 * fp32 input. */
typedef enum { LCE_ACCURATE = 0, LCE_COMPACT = 1 } lce_acc_policy;

/* Output flags (the pages' compute_input_grad / compute_linear_weight_grad /
 * compute_linear_bias_grad, plus the per-row argmax of the logits).
 * LCE_ACCUMULATE adds the gradients to what grad_X / grad_W / grad_b hold
 * (beta = 1) instead of overwriting them, each element rounded once,
 * out = round(out + new): the gradient goes straight into its destination
 * with no separate accumulation pass (Liger-Kernel issue #343, on saving the
 * gradient into the input's .grad directly).  With N == 0 the buffers are
 * left as they are. */
enum {
  LCE_GRAD_X = 1u,
  LCE_GRAD_W = 2u,
  LCE_GRAD_B = 4u,
  LCE_ARGMAX = 8u,
  LCE_ACCUMULATE = 16u
};

/* Special chunk_rows values (torch.nn.LinearCrossEntropyOptions page:
 * chunking_method "aspect_ratio", "aspect_ratio:N", and no chunking). */
#define LCE_CHUNK_ASPECT_RATIO 0   /* next_pow2(ceil(N / ceil(V / D))) rows,
                                      divided by chunk_divisor (floor, >= 1) */
#define LCE_CHUNK_ALL (-1)         /* one chunk of N rows */

/* Problem description, fixed at lce_create.  Enum-typed fields are int32. */
typedef struct {
  int64_t N;             /* rows (batch x sequence, folded) >= 0 */
  int64_t D;             /* in_features >= 1 */
  int64_t V;             /* classes >= 1 */
  int64_t ignore_index;  /* rows with this target are ignored (default -100) */
  int64_t chunk_rows;    /* > 0 rows per chunk, or LCE_CHUNK_* */
  int32_t dtype;         /* lce_dtype of X, W, b and of the gradients */
  int32_t acc_dtype;     /* LCE_F32, or equal to dtype (non-mixed) */
  int32_t has_bias;      /* 0 or 1 */
  int32_t reduction;     /* lce_reduction */
  int32_t acc_policy;    /* lce_acc_policy */
  uint32_t flags;        /* LCE_GRAD_* | LCE_ARGMAX | LCE_ACCUMULATE */
  int64_t chunk_divisor; /* "aspect_ratio:N" with LCE_CHUNK_ASPECT_RATIO: the
                            N >= 1 (0 is read as 1); ignored otherwise */
  int64_t group_rows;    /* ACCURATE with 16-bit inputs only: at most this
                            many rows of dL are held for one grad_W GEMM
                            (rounded down to whole chunks, at least one
                            chunk).  0 = up to 4 D / sizeof(element) rows.
                            A value <= the chunk rows gives one chunk per
                            group: the per-chunk path with an fp32 V x D
                            accumulator carried across chunks.  Ignored by
                            COMPACT, fp32 inputs and non-mixed layouts.
                            An implementation choice (memory against
                            speed), not an option of the pages. */
} lce_desc;

/* Buffers of one call.  All pointers are device pointers. */
typedef struct {
  const void* X;             /* [N, D] dtype */
  const void* W;             /* [V, D] dtype */
  const void* b;             /* [V] dtype; NULL iff has_bias == 0 */
  const int64_t* targets;    /* [N] int64 */
  const float* grad_output;  /* LCE_NONE only: NULL -> loss-only forward
                                (no gradients); non-NULL -> [N] per-row
                                upstream gradient, gradients recomputed from
                                the inputs.  Must be NULL for MEAN / SUM. */
  float* loss;               /* MEAN / SUM: [1] fp32.  NONE: [N] fp32, 0 on
                                ignored rows (may be NULL in the NONE
                                backward). */
  void* grad_X;              /* [N, D] dtype, needs LCE_GRAD_X, else ignored */
  void* grad_W;              /* [V, D] dtype, needs LCE_GRAD_W, else ignored */
  void* grad_b;              /* [V] dtype, needs LCE_GRAD_B and has_bias */
  int32_t* argmax;           /* [N] int32, needs LCE_ARGMAX, else ignored:
                                lowest class index attaining the row max */
  int64_t* n_valid;          /* [1] int64 or NULL: rows that count */
  int64_t* n_bad;            /* [1] int64 or NULL: rows whose target is
                                outside [0, V) and not ignore_index */
  float grad_scale;          /* MEAN / SUM: the upstream gradient of the
                                scalar loss, folded into the gradients
                                (1.0 for a plain backward) */
  int32_t reserved;          /* set to 0 */
  const float* class_weight; /* [V] fp32 per-class weights, or NULL.  The
                                PyTorch module source
                                torch/nn/modules/linear_cross_entropy.py,
                                _ChunkContext's negative target weight: a
                                counted row weighs class_weight[target] in
                                its loss and gradient (NONE: loss[n] is the
                                weighted row loss); MEAN divides by the sum
                                of the counted rows' weights, NaN when that
                                sum is 0.  NULL weighs every class 1. */
} lce_io;

/* Validate `d`, resolve the chunk size and build a handle.  Host only.
 * The validation follows the PyTorch module source
 * torch/nn/modules/linear_cross_entropy.py (_ChunkContext.build), the chunk
 * size the torch.nn.LinearCrossEntropyOptions page (batch_chunk_size,
 * chunking_method "aspect_ratio").
 * Errors: INVALID_ARG (N < 0, D < 1, V < 1, chunk_rows < -1, group_rows < 0, bad
 * acc_policy / has_bias, unknown flag bits, NULL pointers), DTYPE,
 * UNSUPPORTED (a reduction outside lce_reduction, the module source's
 * NotImplementedError; acc_dtype neither LCE_F32 nor dtype; D not a multiple
 * of 8 for bf16 / fp16 or 4 for fp32; the size limits above).  LCE_GRAD_B
 * without a bias is INVALID_ARG. */
LCE_API lce_status lce_create(const lce_desc* d, lce_handle** out);

/* Bytes of device workspace lce_forward_backward needs (host only).  An
 * implementation entry with no counterpart on the pages (their op allocates
 * its scratch itself); the layout is private.  Errors: INVALID_ARG (NULL). */
LCE_API lce_status lce_workspace_size(const lce_handle* h, size_t* bytes);

/* The resolved rows per chunk (0 when N == 0) and the chunk count (host
 * only): the torch.nn.LinearCrossEntropyOptions page's batch_chunk_size as
 * resolved by its chunking_method.  Either output may be NULL.  Errors:
 * INVALID_ARG (NULL handle). */
LCE_API lce_status lce_chunk_info(const lce_handle* h, int64_t* chunk_rows,
                          int64_t* n_chunks);

/* Enqueue the whole chunked forward+backward on `stream`: the batch-chunked
 * accumulator of the PyTorch module source
 * torch/nn/modules/linear_cross_entropy.py, with the weight, input and bias
 * gradients of the PyTorch commit "Fix NJT linear_backward() memory usage"
 * (linear_backward: grad_input = dL W, grad_weight = dL^T X,
 * grad_bias = column sums of dL).
 *
 * Per-row weight g_n (the negated neg_weight_target of the pages), with
 * w_n = class_weight[t_n] (1 without class weights) on counted rows:
 *   MEAN: grad_scale w_n / sum of the counted rows' w (NaN on every row when
 *         that sum is 0, so the loss and every gradient are NaN);
 *   SUM:  grad_scale w_n;
 *   NONE: grad_output[n] w_n (backward only).
 * Ignored rows and rows with out-of-range targets have g_n = 0, loss 0 and a
 * zero grad_X row.  With N == 0, MEAN gives a NaN loss, SUM a zero loss, and
 * grad_W / grad_b are filled with zeros.
 *
 * NaN in X, W or b propagates as in IEEE arithmetic on the definition: a
 * row with a NaN logit has a NaN loss (0 if it is not counted) and a NaN
 * grad_X row, and, since its dL enters every sum over rows (as 0 * NaN on a
 * row that is not counted), NaN in every element of grad_W and grad_b.  The
 * argmax of a row whose logits are all NaN is 0; with some NaN logits it is
 * a valid class, otherwise unspecified.  lce_ce_inplace likewise: a row
 * holding a NaN logit gets a NaN loss and a NaN gradient row.  A -inf logit
 * (a class masked with a -inf bias here, or a -inf logit given to
 * lce_ce_inplace) is a softmax entry of exactly 0: the loss stays finite
 * unless the target's own logit is -inf, and its gradient entries are 0.
 *
 * `workspace` is a device buffer of at least lce_workspace_size bytes,
 * 256-byte aligned; its contents on entry are irrelevant and on return are
 * unspecified.  Calls that share a workspace or outputs must be ordered on
 * one stream.  The handle itself is read-only here, so host threads may share
 * it, except while the timing hook below is enabled (its event pool is not
 * locked).  Errors: INVALID_ARG (NULL required pointer, grad_output set
 * for MEAN / SUM, grad_b requested without bias), WORKSPACE, HIP. */
LCE_API lce_status lce_forward_backward(lce_handle* h, const lce_io* io,
                                void* workspace, size_t ws_bytes,
                                void* stream);

/* out[r][c] = in[r][c] * scale[r * scale_stride] for r < rows, c < cols
 * (dense row-major, row stride cols), in fp32 and rounded to `dtype` (LCE_F32,
 * LCE_BF16 or LCE_F16) to nearest-even; in == out scales in place.  `scale` is a
 * device pointer, so an upstream gradient never travels to the host:
 * scale_stride 0 applies one scalar to everything, 1 one value per row.
 * This is the backward of the ops whose gradients are formed in the forward:
 * the scalar reductions of the PyTorch module source
 * torch/nn/modules/linear_cross_entropy.py (stored gradients times the
 * incoming scalar gradient, in place, or into new buffers when
 * allow_retain_graph is set) and the in-place cross-entropy of Liger-Kernel
 * issue #343 (its gradient times the incoming gradient).  in and out 16-byte
 * aligned; with scale_stride != 0, cols a multiple of 8 (16-bit) or 4 (fp32).
 * Errors: INVALID_ARG (negative sizes or stride, NULL pointer with work to
 * do), DTYPE, UNSUPPORTED (alignment), HIP. */
LCE_API lce_status lce_scale(const void* in, void* out, int32_t dtype, int64_t rows,
                             int64_t cols, const float* scale, int64_t scale_stride,
                             void* stream);

/* Release the handle (NULL is accepted).  Host only; an implementation
 * entry (the pages' op has no handle).  Always LCE_OK. */
LCE_API lce_status lce_destroy(lce_handle* h);

/* Bytes of device workspace for lce_ce_inplace on N rows (host only): four
 * N-element row arrays and three counters.  An implementation entry (the
 * pages' kernel allocates nothing here, the caller's buffer replaces torch's
 * allocator).  Errors: INVALID_ARG (NULL, N < 0, V < 1). */
LCE_API lce_status lce_ce_workspace_size(int64_t N, int64_t V, size_t* bytes);

/* Standalone softmax cross-entropy on precomputed fp32 logits [N, V]
 * (row-major, row stride V, 4-byte aligned, any V >= 1), enqueued on
 * `stream` (Liger-Kernel issue #343: the loss, with the gradient written over
 * the logits).  Writes the loss (MEAN / SUM: loss[1]; NONE: loss[N]) and
 * overwrites `logits` in place with the gradient g_n (softmax - onehot), g_n
 * as for lce_forward_backward with grad_output = grad_scale on every counted
 * row for NONE.  class_weight ([V] fp32 or NULL) weighs rows as in lce_io.
 * n_valid may be NULL.  Errors: INVALID_ARG (N < 0, V < 1, NULL pointers),
 * UNSUPPORTED (a reduction outside lce_reduction, logits not 4-byte
 * aligned, N or V above 2^31 - 1), WORKSPACE, HIP.  Rows of up to 153600
 * classes are held on chip and read from memory once; longer rows are read
 * twice. */
LCE_API lce_status lce_ce_inplace(float* logits, const int64_t* targets,
                          const float* class_weight, int64_t N,
                          int64_t V, int64_t ignore_index, int32_t reduction,
                          float grad_scale, float* loss, int64_t* n_valid,
                          void* workspace, size_t ws_bytes, void* stream);

/* Most rows lce_ce_inplace_noalloc accepts (its static scratch: 16 MiB and
 * 256 bytes per device). */
#define LCE_CE_NOALLOC_MAX_ROWS (1LL << 20)

/* lce_ce_inplace without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * kernels as lce_ce_inplace; its scratch is a static device array of the
 * library, one per GPU, that lives until the process ends.  It calls no
 * hipMalloc / hipFree; the first call on a device looks the array's address
 * up (hipGetSymbolAddress).  Every call on one GPU shares that GPU's array,
 * so calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe.  Nothing in the array needs clearing between calls.
 * Errors: as lce_ce_inplace, plus UNSUPPORTED for N > LCE_CE_NOALLOC_MAX_ROWS
 * (the reason is in lce_last_error) and HIP if the address lookup fails. */
LCE_API lce_status lce_ce_inplace_noalloc(float* logits, const int64_t* targets,
                                          const float* class_weight, int64_t N, int64_t V,
                                          int64_t ignore_index, int32_t reduction,
                                          float grad_scale, float* loss, int64_t* n_valid,
                                          void* stream);

/* Kernel classes of lce_forward_backward, for the timing hook below. */
enum {
  LCE_K_PREP = 0,       /* target counts, row weights, per-row references */
  LCE_K_LOGITS = 1,     /* logits GEMM with the fused softmax-statistics epilogue */
  LCE_K_COMBINE = 2,    /* per-row log-sum-exp, loss, argmax */
  LCE_K_FINALIZE = 3,   /* dL = g (softmax - onehot) in place, dL^T, bias partials */
  LCE_K_GEMM_X = 4,     /* grad_X = dL . W (split-K partials) */
  LCE_K_SPLIT_SUM = 5,  /* split-K reduction into grad_X */
  LCE_K_TRANSPOSE = 6,  /* W^T once per call (fp32 inputs with grad_X); X^T
                           of a grad_W group once per group when the group's
                           dL stays in T (16-bit inputs), else X_chunk^T per
                           chunk beside the staged dL^T */
  LCE_K_GEMM_W = 7,     /* grad_W += dL^T . X_chunk */
  LCE_K_BIAS = 8,       /* grad_b reduction */
  LCE_K_LOSS = 9,       /* final loss reduction, zero fills */
  LCE_K_REPAIR = 10,    /* bf16 gradients: the gated recompute of a chunk with
                           a row whose reference was too low (logits GEMM and
                           combine; empty launches when no row needs it) */
  LCE_K_COUNT = 11
};

/* Timing hook for benchmarks (an implementation entry: the pages measure
 * with a profiler, Liger-Kernel issue #343's proton run).  While enabled, every launch of a kernel class
 * whose bit (1u << LCE_K_*) is in `kernel_mask` is bracketed by two
 * hipEventRecord calls on the call's stream (events come from a fixed pool
 * of 4096 pairs created here; launches beyond the pool are not timed, and
 * the next lce_timing_read says so).  mask 0 disables the hook and releases
 * the events.  Host only; HIP errors -> LCE_ERR_HIP. */
LCE_API lce_status lce_timing_enable(lce_handle* h, uint32_t kernel_mask);

/* Wait for the recorded events, then write per-class totals since the last
 * read: ms[k] (milliseconds) and launches[k] for k < LCE_K_COUNT (either
 * pointer may be NULL), and restart the count.  If launches of a timed class
 * found the pool full since the last read, the totals cover the timed ones
 * only and the call returns LCE_ERR_UNSUPPORTED (lce_last_error gives the
 * count). */
LCE_API lce_status lce_timing_read(lce_handle* h, double* ms, int64_t* launches);

/* Static, human-readable name of a status code (an implementation entry; the
 * pages raise Python exceptions instead of returning codes). */
LCE_API const char* lce_status_string(lce_status s);

/* Text of the last HIP error seen by this thread's calls, or of the last
 * size refusal of lce_ce_inplace_noalloc ("" if none); an implementation
 * entry that complements the status codes. */
LCE_API const char* lce_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
