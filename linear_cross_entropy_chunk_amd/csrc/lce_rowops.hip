// Row-wise and memory-bound kernels of the chunked linear-cross-entropy path:
// target preparation, the per-row combine of the tile statistics, the in-place
// finalize of the logits gradient, padded transposes, deterministic
// reductions, and the standalone softmax cross-entropy that overwrites its
// logits with the gradient.
//
// Sources: torch/nn/modules/linear_cross_entropy.py (_ChunkContext._mask,
// corrected_target and neg_weight_target for the row weights; the chunk loop's
// amax / sumexp / log / "output -=" steps for the loss; the in-place
// softmax * weight step and the one-hot corrections for the gradient; the
// empty-mean NaN fill) and Liger-Kernel issue #343 (cross entropy computed
// and its gradient written over the logits in one kernel).
#include "lce_kernels.h"
#include "lce_device.h"

#include <math.h>

namespace lce {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ float to_f32(_Float16 h) { return static_cast<float>(h); }
template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float f) {
  return static_cast<_Float16>(f);
}
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// ------------------------------------------------------------ target prep
// One workgroup: the mean's denominator must be known before any row weight.
// The weight sum is formed in float64 in a fixed order (per thread, then the
// wave's butterfly, then the waves in index order), so it is deterministic.
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void k_prep(
    const int64_t* __restrict__ t, int N, int V, int64_t ign, int reduction,
    float grad_scale, const float* __restrict__ upstream, const float* __restrict__ cw,
    int* __restrict__ tc, float* __restrict__ g, float* __restrict__ wrow,
    int64_t* __restrict__ counts, int64_t* n_valid_out, int64_t* n_bad_out,
    float* __restrict__ dl_scale) {
  __shared__ long long s_valid[kPrepThreads / 64], s_bad[kPrepThreads / 64];
  __shared__ double s_w[kPrepThreads / 64];
  __shared__ float s_gmax[kPrepThreads / 64];
  __shared__ long long tot[2];
  __shared__ double wtot;
  long long cv = 0, cb = 0;
  double sw = 0.0;
  for (int n = threadIdx.x; n < N; n += kPrepThreads) {
    const int64_t x = t[n];
    const bool ignored = x == ign;
    const bool bad = !ignored && (x < 0 || x >= V);
    const bool valid = !ignored && !bad;
    cv += valid ? 1 : 0;
    cb += bad ? 1 : 0;
    if (valid) sw += cw ? static_cast<double>(cw[x]) : 1.0;
  }
  for (int o = 32; o > 0; o >>= 1) {
    cv += __shfl_xor(cv, o);
    cb += __shfl_xor(cb, o);
    sw += __shfl_xor(sw, o);
  }
  if ((threadIdx.x & 63) == 0) {
    s_valid[threadIdx.x >> 6] = cv;
    s_bad[threadIdx.x >> 6] = cb;
    s_w[threadIdx.x >> 6] = sw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long a = 0, b = 0;
    double w = 0.0;
    for (int k = 0; k < kPrepThreads / 64; ++k) {
      a += s_valid[k];
      b += s_bad[k];
      w += s_w[k];
    }
    tot[0] = a;
    tot[1] = b;
    wtot = w;
    counts[0] = a;
    counts[1] = b;
    counts[2] = __double_as_longlong(w);
    if (n_valid_out) *n_valid_out = a;
    if (n_bad_out) *n_bad_out = b;
  }
  __syncthreads();
  const double d = wtot;
  // reduction codes follow lce.h: 0 mean, 1 sum, 2 none
  const bool mean_nan = reduction == 0 && d == 0.0;
  const double gmean = d != 0.0 ? static_cast<double>(grad_scale) / d : 0.0;
  float gmax = 0.0f;                     // largest finite |g|
  for (int n = threadIdx.x; n < N; n += kPrepThreads) {
    const int64_t x = t[n];
    const bool valid = x != ign && x >= 0 && x < V;
    tc[n] = valid ? static_cast<int>(x) : -1;
    const float wn = valid ? (cw ? cw[x] : 1.0f) : 0.0f;
    if (wrow) wrow[n] = wn;
    float gn;
    if (mean_nan) gn = NAN;
    else if (!valid) gn = 0.0f;
    else if (reduction == 0) gn = static_cast<float>(gmean * wn);
    else if (reduction == 1) gn = grad_scale * wn;
    else gn = (upstream ? upstream[n] : 1.0f) * wn;
    g[n] = gn;
    if (isfinite(gn)) gmax = fmaxf(gmax, fabsf(gn));
  }
  if (dl_scale == nullptr) return;
  for (int o = 32; o > 0; o >>= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, o));
  if ((threadIdx.x & 63) == 0) s_gmax[threadIdx.x >> 6] = gmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.0f;
    for (int k = 0; k < kPrepThreads / 64; ++k) m = fmaxf(m, s_gmax[k]);
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);           // m = f 2^e, f in [0.5, 1)
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    dl_scale[0] = m > 0.0f ? ldexpf(1.0f, -e) : 1.0f;
    dl_scale[1] = m > 0.0f ? ldexpf(1.0f, e) : 1.0f;    // its inverse, exactly
  }
}

// ------------------------------------------------------------ row combine
// Each workgroup (kCbThreads threads) takes kRows consecutive rows, each row
// split into kParts = kCbThreads / kRows parts; part p folds statistics
// blocks p, p + kParts, ... of its row.  The loads of kBatch blocks of a
// part are issued before any is folded, so a thread waits on memory once per
// batch.  The parts are then merged in a fixed order, in two levels: groups
// of kCbGroup consecutive parts, then the groups.  Two layouts:
//   - 32 rows x 32 parts (chunks of at least kCbWideRows rows): a wave's 64
//     lanes are 32 consecutive rows of 2 parts, so each load instruction
//     reads two whole 128-byte lines and every line of the statistics is
//     read by one workgroup only;
//   - 8 rows x 128 parts (smaller chunks, where 32-row workgroups would be
//     too few to keep the loads in flight): each load reads eight 32-byte
//     runs, and the four quarters of a line go to four workgroups, often on
//     different XCDs whose L2s each fetch the whole line.
//   kRef = false: every block has its own max, so sums are rescaled to the
//                 larger max as they merge (an online log-sum-exp);
//   kRef = true:  the blocks share the row's reference, so sums just add.
// The max (and the lowest block attaining it, for the argmax) merges the
// same way in both: a part's max is never NaN (the fold skips NaN block
// maxima, as a comparison with NaN is false).
constexpr int kCbThreads = 1024, kCbGroup = 8, kCbWideRows = 2048;

template <int kRows>
struct CbLayout {
  static constexpr int kParts = kCbThreads / kRows;
  static constexpr int kBatch = kRows == 32 ? 16 : 4;
  static_assert(kRows * kParts == kCbThreads && kParts % kCbGroup == 0, "whole groups");
};

struct Part {
  float m, s;
  int k;
};

template <bool kRef>
__device__ __forceinline__ Part merge(Part a, Part b) {
  Part o;
  const bool take_b = b.m > a.m || (b.m == a.m && b.k < a.k);
  o.m = take_b ? b.m : a.m;
  o.k = take_b ? b.k : a.k;
  if constexpr (kRef) {
    o.s = a.s + b.s;
  } else {
    // A part with max -inf holds sum 0 (blocks wholly past V) or NaN (every
    // logit NaN, which the NaN-skipping max leaves at -inf): its sum is
    // added as it is, so that a NaN reaches the row's result.
    o.s = (a.m > -INFINITY ? a.s * expf(a.m - o.m) : a.s) +
          (b.m > -INFINITY ? b.s * expf(b.m - o.m) : b.s);
  }
  return o;
}

template <bool kRef, int kRows>
__device__ __forceinline__ Part fold_row(const float* __restrict__ mp,
                                         const float* __restrict__ sp, int64_t ldp, int n_vt,
                                         int n, int p) {
  constexpr int kCbParts = CbLayout<kRows>::kParts, kCbBatch = CbLayout<kRows>::kBatch;
  Part a{-INFINITY, 0.0f, 0x7fffffff};
  for (int k0 = p; k0 < n_vt; k0 += kCbBatch * kCbParts) {
    float mb[kCbBatch], sb[kCbBatch];
#pragma unroll
    for (int u = 0; u < kCbBatch; ++u) {
      const int k = k0 + u * kCbParts;
      mb[u] = k < n_vt ? mp[k * ldp + n] : -INFINITY;
      sb[u] = k < n_vt ? sp[k * ldp + n] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kCbBatch; ++u) {
      const float mk = mb[u];
      if constexpr (kRef) {
        if (mk > a.m) {
          a.m = mk;
          a.k = k0 + u * kCbParts;
        }
        a.s += sb[u];
      } else if (mk > a.m) {
        a.s = a.s * expf(a.m - mk) + sb[u];
        a.m = mk;
        a.k = k0 + u * kCbParts;
      } else {
        // blocks with max -inf: sum 0 (wholly past V) or NaN (all NaN)
        a.s += mk > -INFINITY ? sb[u] * expf(mk - a.m) : sb[u];
      }
    }
  }
  return a;
}

// Every part of the workgroup's rows folded and merged; part 0 of row r gets
// the row's (max, sum, lowest block of the max).  Returns false for threads
// that hold no merged row.
template <bool kRef, int kRows>
__device__ __forceinline__ bool combine_parts(const float* __restrict__ mp,
                                              const float* __restrict__ sp, int64_t ldp,
                                              int n_vt, int rows, int& n, Part& out) {
  constexpr int kCbRows = kRows, kCbParts = CbLayout<kRows>::kParts;
  __shared__ float sm[kCbParts][kCbRows], ss[kCbParts][kCbRows];
  __shared__ int sk[kCbParts][kCbRows];
  const int r = threadIdx.x % kCbRows, p = threadIdx.x / kCbRows;
  n = blockIdx.x * kCbRows + r;
  const Part a = n < rows ? fold_row<kRef, kRows>(mp, sp, ldp, n_vt, n, p)
                          : Part{-INFINITY, 0.0f, 0x7fffffff};
  sm[p][r] = a.m;
  ss[p][r] = a.s;
  sk[p][r] = a.k;
  __syncthreads();
  if (p % kCbGroup == 0) {
    Part g{sm[p][r], ss[p][r], sk[p][r]};
    for (int q = p + 1; q < p + kCbGroup; ++q) g = merge<kRef>(g, Part{sm[q][r], ss[q][r], sk[q][r]});
    sm[p][r] = g.m;
    ss[p][r] = g.s;
    sk[p][r] = g.k;
  }
  __syncthreads();
  if (p != 0 || n >= rows) return false;
  Part t{sm[0][r], ss[0][r], sk[0][r]};
  for (int q = kCbGroup; q < kCbParts; q += kCbGroup) t = merge<kRef>(t, Part{sm[q][r], ss[q][r], sk[q][r]});
  out = t;
  return true;
}

// The row's argmax from the partials of the block holding its max.  No
// block is chosen only if every block maximum is NaN (NaN-skipping maxima
// leave -inf and no class), and a block with no class holds 0x7fffffff:
// such a row, whose every logit is NaN, gets class 0, the first NaN, so the
// result is always a valid class.
__device__ __forceinline__ int row_argmax(const int* __restrict__ ip, int64_t ldp, int n_vt,
                                          int k, int n) {
  const int a = ip[static_cast<int64_t>(k < n_vt ? k : 0) * ldp + n];
  return a == 0x7fffffff ? 0 : a;
}

template <int kRows>
__global__ __launch_bounds__(kCbThreads) void k_row_combine(
    const float* __restrict__ mp, const float* __restrict__ sp, const int* __restrict__ ip,
    int64_t ldp, int n_vt, const float* __restrict__ zt, const int* __restrict__ tc,
    const float* __restrict__ wrow, int rows, float* __restrict__ lse,
    float* __restrict__ loss_rows, int* __restrict__ amax) {
  int n;
  Part t;
  if (!combine_parts<false, kRows>(mp, sp, ldp, n_vt, rows, n, t)) return;
  const float L = t.m + logf(t.s);
  lse[n] = L;
  loss_rows[n] = tc[n] >= 0 ? (wrow ? wrow[n] : 1.0f) * (L - zt[n]) : 0.0f;
  if (amax) amax[n] = row_argmax(ip, ldp, n_vt, t.k, n);
}

// ---------------------------------------------- one-reference plan (bf16)
// The reference of row n is its target logit, so that T(n, v) = exp(z - ref)
// holds the softmax up to the row factor 1/S, and the target entry sits at 1.
// One wave per row: lanes over 16-byte vectors of the row, then the wave's
// butterfly (a fixed order).  The first nflags threads clear the repair
// flags of the call's chunks.
template <typename T>
__global__ __launch_bounds__(256) void k_target_logit(
    const T* __restrict__ X, int64_t ldx, const T* __restrict__ W, int64_t ldw,
    const T* __restrict__ bias, const int* __restrict__ tc, int N, int D,
    float* __restrict__ rref, int* __restrict__ flags, int nflags) {
  constexpr int kVec = 16 / sizeof(T);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid < nflags) flags[gid] = 0;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);     // uniform per wave
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const int t = tc[n];
  if (t < 0) {
    // no target: exp(z - inf) = 0 leaves the row's T at 0
    if (lane == 0) rref[n] = INFINITY;
    return;
  }
  const T* x = X + static_cast<int64_t>(n) * ldx;
  const T* w = W + static_cast<int64_t>(t) * ldw;
  float acc = 0.0f;
  for (int d = lane * kVec; d < D; d += 64 * kVec) {
    const i32x4_t xa = *reinterpret_cast<const i32x4_t*>(x + d);
    const i32x4_t wa = *reinterpret_cast<const i32x4_t*>(w + d);
    const T* xe = reinterpret_cast<const T*>(&xa);
    const T* we = reinterpret_cast<const T*>(&wa);
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc += to_f32(xe[e]) * to_f32(we[e]);
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) rref[n] = acc + (bias ? to_f32(bias[t]) : 0.0f);
}

// The combine of the one-reference plan: the blocks' sums share the row's
// reference, so they add without rescaling; the row max only checks the
// reference (and gives the argmax).
template <typename T, int kRows>
__global__ __launch_bounds__(kCbThreads) void k_row_combine_ref(
    const float* __restrict__ mp, const float* __restrict__ sp, const int* __restrict__ ip,
    int64_t ldp, int n_vt, const float* __restrict__ zt, const int* __restrict__ tc,
    const float* __restrict__ wrow, const float* __restrict__ g, int rows,
    float* __restrict__ rref, T* __restrict__ Tm, int64_t tps, float* __restrict__ loss_rows,
    float* __restrict__ beta, int* __restrict__ amax, int* flag, int flag_rows,
    const int* gate) {
  // the repair's combine: a workgroup's rows share one flag (flag_rows is a
  // multiple of the workgroup's rows), so the exit is uniform
  if (gate && gate[flag_rows > 0 ? blockIdx.x * kRows / flag_rows : 0] == 0) return;
  int n;
  Part t;
  if (!combine_parts<true, kRows>(mp, sp, ldp, n_vt, rows, n, t)) return;
  const float M = t.m, S = t.s;
  if (amax) amax[n] = row_argmax(ip, ldp, n_vt, t.k, n);
  const int tt = tc[n];
  const float gn = g[n];
  if (tt < 0) {
    loss_rows[n] = 0.0f;
    beta[n] = gn * 0.0f;          // 0, or NaN when the mean has no rows
    return;
  }
  const float ref = rref[n];
  if (M - ref > kRefGap) {
    // exp(z - ref) may overflow, or beta underflow: recompute the chunk with
    // this row's max as its reference
    rref[n] = M;
    flag[flag_rows > 0 ? n / flag_rows : 0] = 1;
    return;
  }
  const float z = zt[n];
  loss_rows[n] = (wrow ? wrow[n] : 1.0f) * (logf(S) + (ref - z));
  beta[n] = gn / S;
  // dL = g (e / S - onehot) = (g / S) (e - S onehot): the target entry takes
  // its fp32 e minus S, rounded once; e is formed as the logits epilogue
  // forms it (one fused multiply-add, then exp2), so it is the e inside S
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(z, kLog2e, -ref * kLog2e));
  Tm[static_cast<int64_t>(tt / kTile) * tps + static_cast<int64_t>(n) * kTile + tt % kTile] =
      from_f32<T>(e - S);
}

// grad_b of the one-reference plan: acc[v] += sum over the chunk's rows of
// beta_n T(n, v), read from T where the logits epilogue and the combine left
// it (T is not rewritten); the last chunk rounds acc into grad_b.  One
// workgroup per 64 classes: 8 lanes of 16 bytes cover the 64 classes of a
// row, 32 row groups take every 32nd row, four rows' loads in flight per
// thread.  Fixed order throughout: each thread's rows in order, then the
// row groups in order.
constexpr int kBcGroups = 32, kBcUnroll = 4;
template <typename T>
__global__ __launch_bounds__(256) void k_bias_cols(const T* __restrict__ Tm, int64_t tps,
                                                   const float* __restrict__ beta, int rows,
                                                   int V, float* __restrict__ acc,
                                                   T* __restrict__ out, int first, int last,
                                                   int accum) {
  constexpr int kVec = 16 / sizeof(T);
  static_assert(kVec * 8 == 64 && 8 * kBcGroups == 256, "64 classes x 32 row groups");
  __shared__ float red[kBcGroups][65];
  const int v0 = blockIdx.x * 64;
  const int cv = threadIdx.x & 7, rg = threadIdx.x >> 3;
  const T* const col = Tm + static_cast<int64_t>(v0 / kTile) * tps + v0 % kTile + cv * kVec;
  float part[kVec] = {};
  for (int n0 = rg; n0 < rows; n0 += kBcGroups * kBcUnroll) {
    i32x4_t raw[kBcUnroll];
    float b[kBcUnroll];
#pragma unroll
    for (int u = 0; u < kBcUnroll; ++u) {
      const int n = n0 + u * kBcGroups;
      raw[u] = n < rows ? *reinterpret_cast<const i32x4_t*>(col + static_cast<int64_t>(n) * kTile)
                        : i32x4_t{0, 0, 0, 0};
      b[u] = n < rows ? beta[n] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBcUnroll; ++u) {
      if (n0 + u * kBcGroups >= rows) break;
      const T* x = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
      for (int e = 0; e < kVec; ++e) part[e] += b[u] * to_f32(x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) red[rg][cv * kVec + e] = part[e];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int v = v0 + threadIdx.x;
  if (v >= V) return;
  float sum = 0.0f;
  for (int q = 0; q < kBcGroups; ++q) sum += red[q][threadIdx.x];
  const float a = (first ? 0.0f : acc[v]) + sum;
  if (last) out[v] = from_f32<T>(accum ? to_f32(out[v]) + a : a);
  else acc[v] = a;
}

// ------------------------------------------------------- in-place finalize
// 64 rows x 64 classes per workgroup; the 64 classes sit in one statistics
// block of kStatCols classes and in one panel of T.  Writes dL over T, dL^T
// into dLt, and column partials.
template <typename T>
__global__ __launch_bounds__(256) void k_finalize(
    T* __restrict__ Tm, int64_t tps, T* __restrict__ dLt, int64_t ldlt,
    const float* __restrict__ mp, int64_t ldp, const float* __restrict__ lse,
    const float* __restrict__ g, const int* __restrict__ tc, int rows, int V,
    int64_t ldgb, float* __restrict__ gbp, const float* __restrict__ dl_scale) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kVecPerRow = 64 / kVec;
  __shared__ float tile[64][65];
  __shared__ float sc[64], gg[64];
  __shared__ int tt[64];
  constexpr int kPer = 64 * kVecPerRow / 256;          // vectors per thread
  const int v0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int k = v0 / kStatCols;
  const int tid = threadIdx.x;
  T* const pan = Tm + static_cast<int64_t>(v0 / kTile) * tps + v0 % kTile;
  const float ds = dl_scale ? dl_scale[0] : 1.0f;     // stored dL = ds * dL
  // The thread's vectors of T are loaded first, so that their latency
  // overlaps the row scales' loads below.  T has room for all 64 rows of
  // the workgroup (the chunk's rows rounded up to 64); rows past the chunk
  // are rewritten as 0.
  i32x4_t raw[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int idx = tid + 256 * u;
    const int rl = idx / kVecPerRow, cv = idx % kVecPerRow;
    raw[u] = *reinterpret_cast<const i32x4_t*>(pan + static_cast<int64_t>(n0 + rl) * kTile +
                                               cv * kVec);
  }
  if (tid < 64) {
    const int n = n0 + tid;
    const bool in = n < rows;
    const float gn = in ? g[n] : 0.0f;
    sc[tid] = in ? gn * expf(mp[static_cast<int64_t>(k) * ldp + n] - lse[n]) : 0.0f;
    gg[tid] = gn;
    tt[tid] = in ? tc[n] : -1;
  }
  __syncthreads();
  const bool stage = dLt != nullptr || gbp != nullptr;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int idx = tid + 256 * u;
    const int rl = idx / kVecPerRow, cv = idx % kVecPerRow;
    const int n = n0 + rl;
    const int vb = v0 + cv * kVec;
    const T* x = reinterpret_cast<const T*>(&raw[u]);
    i32x4_t outv;
    T* y = reinterpret_cast<T*>(&outv);
    const bool nin = n < rows;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const int v = vb + e;
      float d = 0.0f;
      if (nin && v < V) d = sc[rl] * to_f32(x[e]) - (v == tt[rl] ? gg[rl] : 0.0f);
      if (stage) tile[rl][cv * kVec + e] = d;
      y[e] = from_f32<T>(d * ds);
    }
    *reinterpret_cast<i32x4_t*>(pan + static_cast<int64_t>(n) * kTile + cv * kVec) = outv;
  }
  if (dLt == nullptr && gbp == nullptr) return;
  __syncthreads();
  for (int idx = tid; idx < 64 * kVecPerRow; idx += 256) {
    const int vl = idx / kVecPerRow, nv = idx % kVecPerRow;
    i32x4_t outv;
    T* y = reinterpret_cast<T*>(&outv);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float d = tile[nv * kVec + e][vl];
      part += d;
      y[e] = from_f32<T>(d * ds);
    }
    if (dLt) *reinterpret_cast<i32x4_t*>(dLt + static_cast<int64_t>(v0 + vl) * ldlt + n0 + nv * kVec) = outv;
    if (gbp) {
#pragma unroll
      for (int o = 1; o < kVecPerRow; o <<= 1) part += __shfl_xor(part, o);
      if (nv == 0) gbp[static_cast<int64_t>(blockIdx.y) * ldgb + v0 + vl] = part;
    }
  }
}

// ------------------------------------------------------- padded transpose
// kScale (bf16): row r of the input times row_scale[r], rounded once.
template <typename T, bool kScale>
__global__ __launch_bounds__(256) void k_transpose_pad(const T* __restrict__ in, int64_t ldi,
                                                      int rows, int cols, T* __restrict__ out,
                                                      int64_t ldo, int rows_pad,
                                                      const float* __restrict__ row_scale) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kVecPerRow = 64 / kVec;
  __shared__ T tile[64][64 + kVec];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * kVecPerRow; idx += 256) {
    const int rl = idx / kVecPerRow, cv = idx % kVecPerRow;
    const int r = r0 + rl, c = c0 + cv * kVec;
    i32x4_t raw = i32x4_t{0, 0, 0, 0};
    if (r < rows && c < cols) raw = *reinterpret_cast<const i32x4_t*>(in + static_cast<int64_t>(r) * ldi + c);
    T* x = reinterpret_cast<T*>(&raw);
    if constexpr (kScale) {
      if (r < rows) {
        const float f = row_scale[r];
#pragma unroll
        for (int e = 0; e < kVec; ++e) x[e] = from_f32<T>(to_f32(x[e]) * f);
      }
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) tile[rl][cv * kVec + e] = x[e];
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * kVecPerRow; idx += 256) {
    const int cl = idx / kVecPerRow, rv = idx % kVecPerRow;
    const int c = c0 + cl, r = r0 + rv * kVec;
    if (c >= cols || r >= rows_pad) continue;
    i32x4_t outv;
    T* y = reinterpret_cast<T*>(&outv);
#pragma unroll
    for (int e = 0; e < kVec; ++e) y[e] = tile[rv * kVec + e][cl];
    *reinterpret_cast<i32x4_t*>(out + static_cast<int64_t>(c) * ldo + r) = outv;
  }
}

// ---------------------------------------------------- split-K reduction
template <typename T>
__global__ __launch_bounds__(256) void k_sum_splits(const float* __restrict__ parts, int splits,
                                                   int64_t stride, int64_t count4,
                                                   T* __restrict__ out, int accum,
                                                   const float* __restrict__ scale,
                                                   const float* __restrict__ row_scale,
                                                   int cols) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count4) return;
  f32x4_t acc = reinterpret_cast<const f32x4_t*>(parts)[i];
  for (int s = 1; s < splits; ++s) acc += reinterpret_cast<const f32x4_t*>(parts + s * stride)[i];
  if (scale) acc *= scale[0];
  if (row_scale) acc *= row_scale[4 * i / cols];     // cols % 4 == 0: one row per vector
  if constexpr (sizeof(T) == 4) {
    if (accum) acc += reinterpret_cast<const f32x4_t*>(out)[i];
    reinterpret_cast<f32x4_t*>(out)[i] = acc;
  } else {
    uint2* o = reinterpret_cast<uint2*>(out + 4 * i);
    if (accum) {
      uint2 old = *o;
      const T* x = reinterpret_cast<const T*>(&old);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += to_f32(x[e]);
    }
    uint2 pk;
    T* y = reinterpret_cast<T*>(&pk);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = from_f32<T>(acc[e]);
    *o = pk;
  }
}

// ---------------------------------------------------- bias gradient
template <typename T>
__global__ __launch_bounds__(256) void k_bias_reduce(const float* __restrict__ parts, int nparts,
                                                    int64_t ldp, int V, float* __restrict__ acc,
                                                    T* __restrict__ out, int first, int last,
                                                    int accum) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float a = first ? 0.0f : acc[v];
  for (int b = 0; b < nparts; ++b) a += parts[static_cast<int64_t>(b) * ldp + v];
  if (last) out[v] = from_f32<T>(accum ? to_f32(out[v]) + a : a);
  else acc[v] = a;
}

// ---------------------------------------------------- loss reduction
constexpr int kLossThreads = 1024;
__global__ __launch_bounds__(kLossThreads) void k_loss_reduce(const float* __restrict__ lr, int N,
                                                             const int64_t* __restrict__ counts,
                                                             int reduction, float* __restrict__ loss) {
  __shared__ double part[kLossThreads];
  double s = 0.0;
  for (int n = threadIdx.x; n < N; n += kLossThreads) s += static_cast<double>(lr[n]);
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kLossThreads / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double L = part[0];
    if (reduction == 0) {
      const double d = __longlong_as_double(counts[2]);   // sum of the counted rows' weights
      L = d != 0.0 ? L / d : NAN;
    }
    loss[0] = static_cast<float>(L);
  }
}

__global__ void k_fill_zero(i32x4_t* __restrict__ p, int64_t n16, char* __restrict__ tail,
                            int tail_bytes) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n16) p[i] = i32x4_t{0, 0, 0, 0};
  if (i < tail_bytes) tail[i] = 0;
}

// ---------------------------------------------------- scaling
// One 16-byte vector per thread, inside one row when there are rows; the last
// vector of a length that is not a multiple of the vector width goes element
// by element.
template <typename T>
__global__ __launch_bounds__(256) void k_scale(const T* in, T* out, int64_t n, int64_t cols,
                                               const float* __restrict__ scale, int64_t stride) {
  constexpr int kVec = 16 / sizeof(T);
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kVec;
  if (i >= n) return;
  const float f = scale[cols ? (i / cols) * stride : 0];
  if (i + kVec <= n) {
    i32x4_t raw = *reinterpret_cast<const i32x4_t*>(in + i);
    const T* x = reinterpret_cast<const T*>(&raw);
    i32x4_t outv;
    T* y = reinterpret_cast<T*>(&outv);
#pragma unroll
    for (int e = 0; e < kVec; ++e) y[e] = from_f32<T>(to_f32(x[e]) * f);
    *reinterpret_cast<i32x4_t*>(out + i) = outv;
  } else {
    for (int64_t k = i; k < n; ++k) out[k] = from_f32<T>(to_f32(in[k]) * f);
  }
}

// ---------------------------------------------------- standalone CE
// One workgroup per row.  Pass 1 streams the row with 16-byte loads keeping
// an online (max, sum of exp); pass 2 streams it again and overwrites it with
// g_n (softmax - onehot).  The target logit is read before any overwrite.
// Each thread keeps kCeUnroll independent 16-byte loads in flight, so a
// workgroup has 1024 x 8 x 16 bytes outstanding: enough to cover the memory
// latency at the per-CU share of HBM bandwidth.  Rows of any length and any
// 4-byte alignment: the elements before the row's first 16-byte boundary (h
// < 4) and after its last whole vector (r < 4) go one per thread.
constexpr int kCeThreads = 1024;
constexpr int kCeUnroll = 8;
__global__ __launch_bounds__(kCeThreads) void k_ce_rows(float* __restrict__ z, int V,
                                                       const int* __restrict__ tc,
                                                       const float* __restrict__ g,
                                                       const float* __restrict__ wrow,
                                                       float* __restrict__ loss_rows) {
  __shared__ float wm[kCeThreads / 64], wsum[kCeThreads / 64];
  __shared__ float bcast[2];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  float* rowp = z + static_cast<int64_t>(n) * V;
  const int h = min(static_cast<int>((4 - ((reinterpret_cast<uintptr_t>(rowp) >> 2) & 3)) & 3), V);
  const int V4 = (V - h) >> 2;
  const int r = (V - h) & 3;
  f32x4_t* row = reinterpret_cast<f32x4_t*>(rowp + h);
  const int t = tc[n];
  // this thread's single element outside the vectors, if any
  const int xi = tid < h ? tid : (tid < h + r ? h + 4 * V4 + (tid - h) : -1);
  const float xs = xi >= 0 ? rowp[xi] : -INFINITY;
  // The exponentials take the running max as reference, or 0 while it is
  // -inf (every element so far -inf or NaN): -inf elements then add 0 and
  // NaN ones NaN, as they would against the row's own max.
  float m = fmaxf(-INFINITY, xs);
  float s = xi >= 0 ? fast_exp(xs - (m == -INFINITY ? 0.0f : m)) : 0.0f;
  for (int base = tid; base < V4; base += kCeThreads * kCeUnroll) {
    f32x4_t x[kCeUnroll];
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int i = base + u * kCeThreads;
      x[u] = i < V4 ? row[i] : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u)
      mx = fmaxf(mx, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
    if (mx > m) {
      s *= fast_exp(m - mx);                // 0 (or NaN stays NaN) when m was -inf
      m = mx;
    }
    const float ref = m == -INFINITY ? 0.0f : m;
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u)
      if (base + u * kCeThreads < V4)       // padding adds nothing
        s += fast_exp(x[u][0] - ref) + fast_exp(x[u][1] - ref) + fast_exp(x[u][2] - ref) +
             fast_exp(x[u][3] - ref);
  }
  // A thread whose max is -inf holds sum 0 (no elements, or only -inf ones)
  // or NaN (a NaN element, which the NaN-skipping max leaves at -inf): that
  // sum is added as it is, so that a NaN reaches the row's result.
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o), os = __shfl_xor(s, o);
    const float M = fmaxf(m, om);
    s = (m > -INFINITY ? s * fast_exp(m - M) : s) + (om > -INFINITY ? os * fast_exp(om - M) : os);
    m = M;
  }
  if ((tid & 63) == 0) {
    wm[tid >> 6] = m;
    wsum[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = wm[0];
    for (int w = 1; w < kCeThreads / 64; ++w) M = fmaxf(M, wm[w]);
    float S = 0.0f;
    for (int w = 0; w < kCeThreads / 64; ++w)
      S += wm[w] > -INFINITY ? wsum[w] * expf(wm[w] - M) : wsum[w];
    const float L = M + logf(S);
    const float zt = t >= 0 ? rowp[t] : 0.0f;
    loss_rows[n] = t >= 0 ? (wrow ? wrow[n] : 1.0f) * (L - zt) : 0.0f;
    bcast[0] = L;
  }
  __syncthreads();
  const float L = bcast[0];
  const float gn = g[n];
  if (xi >= 0) rowp[xi] = gn * fast_exp(xs - L) - (xi == t ? gn : 0.0f);
  for (int base = tid; base < V4; base += kCeThreads * kCeUnroll) {
    f32x4_t x[kCeUnroll];
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int i = base + u * kCeThreads;
      if (i < V4) x[u] = row[i];
    }
#pragma unroll
    for (int u = 0; u < kCeUnroll; ++u) {
      const int i = base + u * kCeThreads;
      if (i >= V4) continue;
      f32x4_t y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = gn * fast_exp(x[u][e] - L);
        if (h + 4 * i + e == t) y[e] -= gn;
      }
      __builtin_nontemporal_store(y, row + i);
    }
  }
}

// Single-read variant for long rows: the whole row stays on chip, kRegVec
// 16-byte vectors per thread in registers plus a tail of up to kTailVec
// vectors in LDS (copied there straight from memory), so the row is read from
// HBM once and written once.  Max, then exp(x - max) in place with its sum,
// then the gradient g (e / sum - onehot): one exponential per element.  As in
// k_ce_rows, the elements before the row's first 16-byte boundary and after
// its last whole vector (fewer than 4 each) go one per thread.
// kThr threads of kRegVec vectors each: 256 threads (registers only, several
// workgroups per CU), 512 (two waves per SIMD, 256 registers each) or 1024
// (four per SIMD, 128 each); kTailVec vectors of LDS.
template <int kThr, int kRegVec, int kTailVec>
__global__ __launch_bounds__(kThr) void k_ce_rows_onchip(float* __restrict__ z, int V,
                                                              const int* __restrict__ tc,
                                                              const float* __restrict__ g,
                                                              const float* __restrict__ wrow,
                                                              float* __restrict__ loss_rows) {
  __shared__ __attribute__((aligned(16))) f32x4_t tail[kTailVec];
  __shared__ float wred[kThr / 64];
  __shared__ float bcast[2];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* rowp = z + static_cast<int64_t>(n) * V;
  const int h = min(static_cast<int>((4 - ((reinterpret_cast<uintptr_t>(rowp) >> 2) & 3)) & 3), V);
  f32x4_t* row = reinterpret_cast<f32x4_t*>(rowp + h);
  const int V4 = (V - h) >> 2;
  const int r = (V - h) & 3;
  const int nreg = min(V4, kThr * kRegVec);       // vectors held in registers
  const int ntail = V4 - nreg;                          // vectors held in LDS
  const int t = tc[n];
  // this thread's single element outside the vectors, if any
  const int xi = tid < h ? tid : (tid < h + r ? h + 4 * V4 + (tid - h) : -1);

  // The tail, 1 KiB blocks of 64 vectors, one copy instruction each; lanes
  // past the row end read as zero (and are never used).
  const __amdgpu_buffer_rsrc_t rs = dev::make_rsrc(row, static_cast<int64_t>(V4) * 16);
  for (int b = wave; b * 64 < ntail; b += kThr / 64)
    dev::copy16_to_lds(rs, (nreg + b * 64 + lane) * 16, dev::lds_addr(tail + b * 64));
  // Register part: one lane offset, the vector stride in the scalar offset.
  f32x4_t x[kRegVec];
#pragma unroll
  for (int u = 0; u < kRegVec; ++u) {
    const int i = tid + u * kThr;
    const f32x4_t v = __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, u * kThr * 16, 0));
    x[u] = i < nreg ? v : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  float zt = 0.0f;
  if (tid == 0 && t >= 0) zt = rowp[t];
  float xs = xi >= 0 ? rowp[xi] : -INFINITY;
  __builtin_amdgcn_s_waitcnt(dev::waitcnt_vm(0));
  __syncthreads();

  auto block_max = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if (lane == 0) wred[wave] = v;
    __syncthreads();
    if (tid == 0) {
      float r = wred[0];
      for (int w = 1; w < kThr / 64; ++w) r = fmaxf(r, wred[w]);
      bcast[0] = r;
    }
    __syncthreads();
    return bcast[0];
  };
  auto block_sum = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) wred[wave] = v;
    __syncthreads();
    if (tid == 0) {
      float r = 0.0f;
      for (int w = 0; w < kThr / 64; ++w) r += wred[w];
      bcast[1] = r;
    }
    __syncthreads();
    return bcast[1];
  };

  float m = xs;
#pragma unroll
  for (int u = 0; u < kRegVec; ++u)
    m = fmaxf(m, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
  for (int j = tid; j < ntail; j += kThr) {
    const f32x4_t v = tail[j];
    m = fmaxf(m, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  const float M = block_max(m);

  xs = xi >= 0 ? fast_exp(xs - M) : 0.0f;
  float s = xs;
#pragma unroll
  for (int u = 0; u < kRegVec; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[u][e] = fast_exp(x[u][e] - M);       // -inf slots become 0
      s += x[u][e];
    }
  for (int j = tid; j < ntail; j += kThr) {
    f32x4_t v = tail[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = fast_exp(v[e] - M);
      s += v[e];
    }
    tail[j] = v;
  }
  const float S = block_sum(s);
  const float L = M + logf(S);
  if (tid == 0) loss_rows[n] = t >= 0 ? (wrow ? wrow[n] : 1.0f) * (L - zt) : 0.0f;

  const float gn = g[n];
  const float scale = gn / S;
  if (xi >= 0) rowp[xi] = xs * scale - (xi == t ? gn : 0.0f);
  const int tb = t - h;                                 // the target's index in the vectors
#pragma unroll
  for (int u = 0; u < kRegVec; ++u) {
    const int i = tid + u * kThr;
    if (i >= nreg) continue;
    f32x4_t y = x[u] * scale;
    if (tb >= 4 * i && tb < 4 * i + 4) y[tb - 4 * i] -= gn;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, y), rs, tid * 16,
                                           u * kThr * 16, 0);
  }
  for (int j = tid; j < ntail; j += kThr) {
    const int i = nreg + j;
    f32x4_t y = tail[j] * scale;
    if (tb >= 4 * i && tb < 4 * i + 4) y[tb - 4 * i] -= gn;
    __builtin_nontemporal_store(y, row + i);
  }
}

// Short rows: one wave per row, the row in the wave's registers (kVec 16-byte
// vectors per lane, up to 64 kVec vectors), so it is read once and written
// once and the max and the sum need only the wave's own shuffles.  Four rows
// per workgroup.  Head and tail elements outside the vectors as in k_ce_rows.
constexpr int kWaveRows = 4;
template <int kVec>
__global__ __launch_bounds__(64 * kWaveRows) void k_ce_rows_wave(float* __restrict__ z, int N,
                                                                 int V,
                                                                 const int* __restrict__ tc,
                                                                 const float* __restrict__ g,
                                                                 const float* __restrict__ wrow,
                                                                 float* __restrict__ loss_rows) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaveRows + (threadIdx.x >> 6);
  if (n >= N) return;                                   // whole waves: no barrier below
  float* rowp = z + static_cast<int64_t>(n) * V;
  const int h = min(static_cast<int>((4 - ((reinterpret_cast<uintptr_t>(rowp) >> 2) & 3)) & 3), V);
  const int V4 = (V - h) >> 2;
  const int r = (V - h) & 3;
  const __amdgpu_buffer_rsrc_t rs = dev::make_rsrc(rowp + h, static_cast<int64_t>(V4) * 16);
  const int t = tc[n];
  const int xi = lane < h ? lane : (lane < h + r ? h + 4 * V4 + (lane - h) : -1);
  float xs = xi >= 0 ? rowp[xi] : -INFINITY;
  const float zt = t >= 0 ? rowp[t] : 0.0f;
  f32x4_t x[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const f32x4_t v = __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, u * 64 * 16, 0));
    x[u] = lane + 64 * u < V4 ? v : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  float m = xs;
#pragma unroll
  for (int u = 0; u < kVec; ++u)
    m = fmaxf(m, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  xs = xi >= 0 ? fast_exp(xs - m) : 0.0f;
  float s = xs;
#pragma unroll
  for (int u = 0; u < kVec; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[u][e] = fast_exp(x[u][e] - m);                  // padding: exp(-inf) = 0
      s += x[u][e];
    }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) {
    const float L = m + logf(s);
    loss_rows[n] = t >= 0 ? (wrow ? wrow[n] : 1.0f) * (L - zt) : 0.0f;
  }
  const float gn = g[n];
  const float scale = gn / s;
  if (xi >= 0) rowp[xi] = xs * scale - (xi == t ? gn : 0.0f);
  const int tb = t - h;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int i = lane + 64 * u;
    if (i >= V4) continue;
    f32x4_t y = x[u] * scale;
    if (tb >= 4 * i && tb < 4 * i + 4) y[tb - 4 * i] -= gn;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, y), rs, lane * 16,
                                           u * 64 * 16, 0);
  }
}

inline unsigned cdiv_u(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

hipError_t prep_targets(const int64_t* t, int N, int V, int64_t ignore_index, int reduction,
                        float grad_scale, const float* upstream, const float* class_weight,
                        int* tc, float* g, float* wrow, int64_t* counts, int64_t* n_valid_out,
                        int64_t* n_bad_out, float* dl_scale, hipStream_t s) {
  k_prep<<<1, kPrepThreads, 0, s>>>(t, N, V, ignore_index, reduction, grad_scale, upstream,
                                    class_weight, tc, g, wrow, counts, n_valid_out, n_bad_out,
                                    dl_scale);
  return hipGetLastError();
}

hipError_t row_combine(const float* m_part, const float* s_part, const int* i_part, int64_t ldp,
                       int n_vt, const float* zt, const int* tc, const float* wrow, int rows,
                       float* lse, float* loss_rows, int* argmax_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows >= kCbWideRows)
    k_row_combine<32><<<cdiv_u(rows, 32), kCbThreads, 0, s>>>(
        m_part, s_part, i_part, ldp, n_vt, zt, tc, wrow, rows, lse, loss_rows, argmax_out);
  else
    k_row_combine<8><<<cdiv_u(rows, 8), kCbThreads, 0, s>>>(
        m_part, s_part, i_part, ldp, n_vt, zt, tc, wrow, rows, lse, loss_rows, argmax_out);
  return hipGetLastError();
}

// Instantiate a 2-byte or 4-byte kernel for the element type.
#define LCE_BY_ELEM(e, KERNEL_CALL)                        \
  do {                                                     \
    if ((e) == Elem::kBF16) { using T = uint16_t; KERNEL_CALL; } \
    else if ((e) == Elem::kF16) { using T = _Float16; KERNEL_CALL; } \
    else { using T = float; KERNEL_CALL; }                 \
  } while (0)

hipError_t target_logits(Elem e, const void* X, int64_t ldx, const void* W, int64_t ldw,
                         const void* bias, const int* tc, int N, int D, float* rref,
                         int* flags, int nflags, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (nflags > 64 * static_cast<int64_t>(N)) return hipErrorInvalidValue;
  LCE_BY_ELEM(e, (k_target_logit<T><<<cdiv_u(N, 4), 256, 0, s>>>(
                     static_cast<const T*>(X), ldx, static_cast<const T*>(W), ldw,
                     static_cast<const T*>(bias), tc, N, D, rref, flags, nflags)));
  return hipGetLastError();
}

hipError_t row_combine_ref(const float* m_part, const float* s_part, const int* i_part,
                           int64_t ldp, int n_vt, const float* zt, const int* tc,
                           const float* wrow, const float* g, int rows, float* rref, void* Tb,
                           int64_t tps, float* loss_rows, float* beta, int* argmax_out,
                           int* flag, int flag_rows, const int* gate, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (flag_rows < 0 || flag_rows % 256 != 0) return hipErrorInvalidValue;
  uint16_t* Tm = static_cast<uint16_t*>(Tb);
  if (rows >= kCbWideRows)
    k_row_combine_ref<uint16_t, 32><<<cdiv_u(rows, 32), kCbThreads, 0, s>>>(
        m_part, s_part, i_part, ldp, n_vt, zt, tc, wrow, g, rows, rref, Tm, tps, loss_rows, beta,
        argmax_out, flag, flag_rows, gate);
  else
    k_row_combine_ref<uint16_t, 8><<<cdiv_u(rows, 8), kCbThreads, 0, s>>>(
        m_part, s_part, i_part, ldp, n_vt, zt, tc, wrow, g, rows, rref, Tm, tps, loss_rows, beta,
        argmax_out, flag, flag_rows, gate);
  return hipGetLastError();
}

hipError_t bias_cols(const void* Tb, int64_t tps, const float* beta, int rows, int V,
                     float* acc, void* out, bool first, bool last, bool accum, hipStream_t s) {
  if (V <= 0) return hipSuccess;
  k_bias_cols<uint16_t><<<cdiv_u(V, 64), 256, 0, s>>>(static_cast<const uint16_t*>(Tb), tps,
                                                      beta, rows, V, acc,
                                                      static_cast<uint16_t*>(out), first, last,
                                                      accum);
  return hipGetLastError();
}

hipError_t finalize_dlogits(Elem e, void* Tb, int64_t tps, void* dLt, int64_t ldlt,
                            const float* m_part, int64_t ldp, const float* lse, const float* g,
                            const int* tc, int rows, int rows_pad, int V, int V_pad,
                            float* gb_part, const float* dl_scale, hipStream_t s) {
  if (rows_pad <= 0) return hipSuccess;
  const dim3 grid(V_pad / 64, rows_pad / 64);
  LCE_BY_ELEM(e, (k_finalize<T><<<grid, 256, 0, s>>>(static_cast<T*>(Tb), tps,
                                                    static_cast<T*>(dLt), ldlt, m_part, ldp,
                                                    lse, g, tc, rows, V, V_pad, gb_part,
                                                    dl_scale)));
  return hipGetLastError();
}

hipError_t scale(Elem e, const void* in, void* out, int64_t n, int64_t cols,
                 const float* f, int64_t stride, hipStream_t s) {
  const int vec = 16 / elem_size(e);
  const int64_t vecs = (n + vec - 1) / vec;
  const int64_t blocks = (vecs + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  LCE_BY_ELEM(e, (k_scale<T><<<static_cast<unsigned>(blocks), 256, 0, s>>>(
                     static_cast<const T*>(in), static_cast<T*>(out), n, cols, f, stride)));
  return hipGetLastError();
}

hipError_t transpose_pad(Elem e, const void* in, int64_t ldi, int rows, int cols, void* out,
                         int64_t ldo, int rows_pad, hipStream_t s, const float* row_scale) {
  if (rows_pad <= 0 || cols <= 0) return hipSuccess;
  if (row_scale && e != Elem::kBF16) return hipErrorInvalidValue;
  const dim3 grid(cdiv_u(cols, 64), cdiv_u(rows_pad, 64));
  // a bit copy: both 2-byte types go through the uint16_t instance
  if (row_scale)
    k_transpose_pad<uint16_t, true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(in), ldi,
                                                         rows, cols, static_cast<uint16_t*>(out),
                                                         ldo, rows_pad, row_scale);
  else if (elem_size(e) == 2)
    k_transpose_pad<uint16_t, false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(in), ldi,
                                                          rows, cols, static_cast<uint16_t*>(out),
                                                          ldo, rows_pad, nullptr);
  else
    k_transpose_pad<float, false><<<grid, 256, 0, s>>>(static_cast<const float*>(in), ldi, rows,
                                                       cols, static_cast<float*>(out), ldo,
                                                       rows_pad, nullptr);
  return hipGetLastError();
}

hipError_t sum_splits(Elem e, const float* parts, int splits, int64_t stride, int rows,
                      int cols, void* out, bool accum, const float* scale, hipStream_t s,
                      const float* row_scale) {
  const int64_t count4 = static_cast<int64_t>(rows) * cols / 4;
  if (count4 <= 0) return hipSuccess;
  if (row_scale && cols % 4 != 0) return hipErrorInvalidValue;
  LCE_BY_ELEM(e, (k_sum_splits<T><<<cdiv_u(count4, 256), 256, 0, s>>>(
                     parts, splits, stride, count4, static_cast<T*>(out), accum, scale,
                     row_scale, cols)));
  return hipGetLastError();
}

hipError_t bias_grad_reduce(Elem e, const float* parts, int nparts, int64_t ldp, int V,
                            float* acc, void* out, bool first, bool last, bool accum,
                            hipStream_t s) {
  if (V <= 0) return hipSuccess;
  LCE_BY_ELEM(e, (k_bias_reduce<T><<<cdiv_u(V, 256), 256, 0, s>>>(
                     parts, nparts, ldp, V, acc, static_cast<T*>(out), first, last, accum)));
  return hipGetLastError();
}

hipError_t loss_reduce(const float* loss_rows, int N, const int64_t* counts, int reduction,
                       float* loss, hipStream_t s) {
  k_loss_reduce<<<1, kLossThreads, 0, s>>>(loss_rows, N, counts, reduction, loss);
  return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int tail = static_cast<int>(bytes % 16);
  const int64_t work = n16 > tail ? n16 : tail;
  k_fill_zero<<<cdiv_u(work, 256), 256, 0, s>>>(static_cast<i32x4_t*>(p), n16,
                                                static_cast<char*>(p) + n16 * 16, tail);
  return hipGetLastError();
}

hipError_t ce_inplace_rows(float* z, int N, int V, const int* tc, const float* g,
                           const float* wrow, float* loss_rows, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  // Rows of up to 4099 classes go one per wave, in registers (1000 classes:
  // 2.6x the two-pass rate; at 6000-8192 classes a wave of 32 vectors per
  // lane was slower than two passes); rows of 4100 to 153600 classes stay on
  // chip in a workgroup (one HBM read either way: 4100 classes 1.4x, 6000
  // to 50000 classes 3-16% faster than two passes, 8192 classes 5% slower);
  // longer rows stream twice.  A row's vectors number at most V / 4
  // whatever its alignment.
  const int V4 = V / 4;
  const unsigned wave_grid = cdiv_u(N, kWaveRows);
  auto fits = [&](int thr, int reg, int tail) { return V4 >= 1025 && V4 <= thr * reg + tail; };
  if (V4 <= 64 * 4)
    k_ce_rows_wave<4><<<wave_grid, 64 * kWaveRows, 0, s>>>(z, N, V, tc, g, wrow, loss_rows);
  else if (V4 <= 64 * 8)
    k_ce_rows_wave<8><<<wave_grid, 64 * kWaveRows, 0, s>>>(z, N, V, tc, g, wrow, loss_rows);
  else if (V4 <= 64 * 16)
    k_ce_rows_wave<16><<<wave_grid, 64 * kWaveRows, 0, s>>>(z, N, V, tc, g, wrow, loss_rows);
  else if (fits(256, 16, 64))      // registers only: up to 16640 classes
    k_ce_rows_onchip<256, 16, 64><<<N, 256, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  else if (fits(512, 16, 8192))
    k_ce_rows_onchip<512, 16, 8192><<<N, 512, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  else if (fits(512, 32, 8192))
    k_ce_rows_onchip<512, 32, 8192><<<N, 512, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  else if (fits(512, 48, 8192))
    k_ce_rows_onchip<512, 48, 8192><<<N, 512, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  else if (fits(1024, 28, 9728))   // up to 153600 classes: 152 KiB of LDS
    k_ce_rows_onchip<1024, 28, 9728><<<N, 1024, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  else k_ce_rows<<<N, kCeThreads, 0, s>>>(z, V, tc, g, wrow, loss_rows);
  return hipGetLastError();
}

}  // namespace lce
