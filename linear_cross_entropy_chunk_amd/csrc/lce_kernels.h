// Internal launchers shared by the translation units of liblce.so.
// Every launcher only enqueues work on `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

// Element type of X, W, b, the gradients and the exp / dL buffer T.  bf16 and
// fp16 accumulate in fp32.
enum class Elem : int { kF32 = 0, kBF16 = 1, kF16 = 2 };
inline int elem_size(Elem e) { return e == Elem::kF32 ? 4 : 2; }

// Square output tile of every GEMM launch (rows x cols of C per workgroup).
constexpr int kTile = 256;
// Classes per softmax-statistics partial of the logits epilogue (one wave's
// share of a tile's classes).
constexpr int kStatCols = 128;
// Rows per K4 finalize / transpose tile.
constexpr int kSmallTile = 64;

// Layout of the exp / dL buffer T of a chunk (or of a group of chunks): panels
// of kTile classes, each panel [R][kTile] with the rows of every chunk of the
// group back to back; element (n, v) lies at
//   T + (v / kTile) * pstride + n * kTile + v % kTile,   pstride = R * kTile.
// A logits tile (kTile classes x kTile rows) is then 128 KiB (bf16) of
// consecutive memory, and the grad_W GEMM reads the classes of its tile over
// all rows as one contiguous panel.

// kAccumF32 and kFinalOut load the stored fp32 values into the accumulators
// before the K loop and only store at the end; kAccumOut and kFinalAccum read
// their inputs in the epilogue.
enum class EpiMode : int {
  kStoreF32 = 0,     // C = acc                      (fp32 out, e.g. split-K parts)
  kAccumF32 = 1,     // C = C + acc                  (fp32 in/out)
  kFinalOut = 2,     // out = cvt(C_f32 + acc)       (fp32 in, dtype out)
  kStoreOut = 3,     // out = cvt(acc)               (dtype out)
  kAccumOut = 4,     // out = cvt(out + acc)         (dtype in/out)
  kFinalAccum = 5    // out = cvt(out + C_f32 + acc) (fp32 in, dtype in/out; grad_W only)
};

// ---- GEMM (lce_gemm.hip) -------------------------------------------------
// P[m, n] = sum_k A(m, k) B(n, k).  A is stored either [M][lda] with K
// contiguous, or k-major [K][lda] with M contiguous (a_kmajor, bf16 only);
// B likewise with N (not both k-major).  Rows of a k-major operand at or past a_krows (b_krows)
// read as zero.  The result is stored transposed, C[n * ldc + m] (M a
// multiple of 4).  K is split into `splits` ranges of k_split elements (a
// multiple of the stage depth); split s writes C + s * split_stride.
enum class GemmRole : int { kGradX = 0, kGradW = 1 };   // names the kernel in profiles

struct GemmNT {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  int M, N, K;
  int splits; int k_split; int64_t split_stride;
  void* C; int64_t ldc;           // output
  const void* Cin;                // input of the accumulate modes (ld = ldc)
  EpiMode mode;
  int group_m;                    // tile-order grouping along M
  GemmRole role;
  bool a_kmajor, b_kmajor;        // operand layouts (see above)
  int a_krows, b_krows;           // valid k rows of a k-major operand
  // B in the T panel layout (ldb = kTile): the grad_X kernel's B is always
  // T (classes along K); the grad_W kernel's k-major B is T (classes along N).
  int64_t b_pstride;
  // Device scalar that multiplies the product wherever it is written in the
  // element type (modes kStoreOut, kAccumOut, kFinalOut, kFinalAccum; the
  // fp32 modes store it unscaled); null means 1.
  const float* out_scale;
  // Per-column factors n_scale[n] (n < N) that also multiply column n of the
  // product in modes kStoreOut and kAccumOut (grad_X: one factor per batch
  // row); null means 1.
  const float* n_scale;
};
hipError_t gemm_nt(Elem e, const GemmNT& g, hipStream_t s);

// Logits GEMM with the fused softmax-statistics epilogue.  Computes, for the
// chunk's rows n < rows and classes v < V, z[n, v] = X[n] . W[v] + b[v]; per
// block k of kStatCols classes it writes the block max m_part[k][n], the block
// sum of exp(z - ref) s_part[k][n], the lowest class index attaining the
// block max i_part[k][n] (if i_part != null), z[n, tc[n]] into zt[n]
// (tc[n] < 0: none), and when T != null, T(n, v) = exp(z[n, v] - ref)
// rounded to the element type, for v < V_pad (0 beyond V), in the panel
// layout with panel stride tps (T points at the chunk's row 0).
//   ref = m_part[k][n] (the block max) when rref is null;
//   ref = rref[n], one reference per row for all its classes, when rref is
//         set (bf16 with T only).  Rows rows <= n < t_rows of T are then
//         written as 0 (a ragged chunk's padding, read by grad_W's K range).
// With `gate` set the launch is the repair pass of rows whose reference was
// too low: gate[k] is the flag of rows [k gate_rows, (k + 1) gate_rows)
// (gate_rows a multiple of kTile, or 0 for one flag over all rows); the
// launch does nothing unless a flag is set, and then recomputes, with a grid
// of at most one workgroup per CU, the tiles of the flagged rows.
struct LogitsLse {
  const void* X; int64_t ldx;     // chunk rows [rows][D]
  const void* W; int64_t ldw;     // [V][D]
  const void* bias;               // [V] or null
  const int* tc;                  // [rows]
  int rows, V, D;
  void* T; int64_t tps;           // panel layout, or null
  float* m_part; float* s_part; int* i_part; int64_t ldp;   // [V_pad / kStatCols][ldp]
  float* zt;                      // [rows]
  const float* rref;              // [rows] per-row reference, or null
  int t_rows;                     // rows of T written (rref set: >= rows)
  const int* gate;                // null, or the repair flags
  int gate_rows;                  // rows per flag (0: one flag)
};
hipError_t logits_lse(Elem e, const LogitsLse& a, hipStream_t s);

// ---- row-wise kernels (lce_rowops.hip) -------------------------------------
// Target preparation: counts rows, forms corrected targets and row weights.
//   tc[n]   = t[n] if 0 <= t[n] < V and t[n] != ignore_index, else -1
//   w[n]    = class_weight[tc[n]] (1 without class weights) if tc[n] >= 0,
//             else 0; written to wrow when wrow != null
//   g[n]    = per-row weight of the reduction (see lce.h), built from w
// counts[0] = n_valid, counts[1] = n_bad (also copied to the optional outs),
// counts[2] = the bits of the double sum of w (the mean's denominator).
// dl_scale (if not null): [0] = 2^k with 2^k max_n |g[n]| in [0.5, 1) (1 when
// every g is 0 or not finite), the factor that keeps dL inside fp16's range;
// [1] = 2^-k.
hipError_t prep_targets(const int64_t* t, int N, int V, int64_t ignore_index,
                        int reduction, float grad_scale, const float* upstream,
                        const float* class_weight, int* tc, float* g, float* wrow,
                        int64_t* counts, int64_t* n_valid_out, int64_t* n_bad_out,
                        float* dl_scale, hipStream_t s);

// Row combine over the n_vt statistics blocks of a chunk: lse[n] (chunk-local),
// loss_rows[n] = w[n] (lse - zt) (0 if tc < 0; w = wrow[n], 1 when wrow is
// null), argmax_out[n] if non-null.
hipError_t row_combine(const float* m_part, const float* s_part, const int* i_part,
                       int64_t ldp, int n_vt, const float* zt, const int* tc,
                       const float* wrow, int rows, float* lse, float* loss_rows,
                       int* argmax_out, hipStream_t s);

// Per-row reference of the one-reference plan (bf16): rref[n] = X[n] .
// W[tc[n]] + b[tc[n]] in fp32 (the target logit, up to rounding order), +inf
// where tc[n] < 0; also clears flags[0 .. nflags) (nflags <= 64 N).
hipError_t target_logits(Elem e, const void* X, int64_t ldx, const void* W, int64_t ldw,
                         const void* bias, const int* tc, int N, int D, float* rref,
                         int* flags, int nflags, hipStream_t s);

// Row combine of the one-reference plan (bf16): for the chunk's rows, with
// S = sum_k s_part[k][n] (sums of exp(z - rref[n])) and M the row max,
//   - tc < 0: loss_rows 0, beta = g * 0;
//   - M - rref > kRefGap: the reference is too far below the row max (a row
//     whose loss is then above kRefGap nats): rref[n] = M and its flag is set,
//     so that the gated repair pass recomputes the flag's rows with that row's max;
//   - otherwise loss_rows = w (log S + rref - zt), beta = g / S, and the
//     target entry of T becomes exp(zt - rref) - S, so that
//     dL[n][v] = beta[n] T(n, v) (softmax times S, minus S at the target).
// argmax_out as row_combine.  flag[k] belongs to rows [k flag_rows,
// (k + 1) flag_rows) (flag_rows a multiple of 256, or 0 for one flag over all
// rows).  With `gate` (the same flags) the launch is the repair's combine:
// rows whose flag is clear are left alone.
constexpr float kRefGap = 40.0f;
hipError_t row_combine_ref(const float* m_part, const float* s_part, const int* i_part,
                           int64_t ldp, int n_vt, const float* zt, const int* tc,
                           const float* wrow, const float* g, int rows, float* rref,
                           void* T, int64_t tps, float* loss_rows, float* beta,
                           int* argmax_out, int* flag, int flag_rows, const int* gate,
                           hipStream_t s);

// grad_b of the one-reference plan (bf16), one chunk: for v < V,
// acc[v] = (first ? 0 : acc[v]) + sum_{n < rows} beta[n] T(n, v); with last,
// out[v] = cvt(acc (+ out[v] if accum)) instead.  T in the panel layout.
hipError_t bias_cols(const void* T, int64_t tps, const float* beta, int rows, int V,
                     float* acc, void* out, bool first, bool last, bool accum, hipStream_t s);

// In-place finalize: T(n, v) <- dL = g_n (T * exp(m_part[v/kStatCols][n] - lse_n)
// - [v == tc_n]) for n < rows_pad, v < V_pad (0 where n >= rows or v >= V), T
// in the panel layout with panel stride tps; optionally writes dLt[v][n]
// (ld = ldlt) and per-64-row column partials gb_part[n/64][v] (ld = V_pad).
// dL is stored times dl_scale[0] when dl_scale is not null (the partials are
// not scaled).
hipError_t finalize_dlogits(Elem e, void* T, int64_t tps, void* dLt, int64_t ldlt,
                            const float* m_part, int64_t ldp, const float* lse,
                            const float* g, const int* tc, int rows, int rows_pad,
                            int V, int V_pad, float* gb_part, const float* dl_scale,
                            hipStream_t s);

// out[c][r] = r < rows ? in[r][c] : 0 for r < rows_pad, c < cols; with
// row_scale (bf16 only) in[r][c] * row_scale[r], rounded once.
hipError_t transpose_pad(Elem e, const void* in, int64_t ldi, int rows, int cols,
                         void* out, int64_t ldo, int rows_pad, hipStream_t s,
                         const float* row_scale = nullptr);

// out[r][c] = cvt(f_r * sum_s parts[s][r][c] (+ out[r][c] if accum)) for
// r < rows, c < cols (ld = cols), f_r = scale[0] (1 when scale is null) times
// row_scale[r] (1 when row_scale is null).
hipError_t sum_splits(Elem e, const float* parts, int splits, int64_t stride,
                      int rows, int cols, void* out, bool accum, const float* scale,
                      hipStream_t s, const float* row_scale = nullptr);

// acc[v] = (first ? 0 : acc[v]) + sum_b parts[b][v]; if last:
// out[v] = cvt(acc (+ out[v] if accum)).
hipError_t bias_grad_reduce(Elem e, const float* parts, int nparts, int64_t ldp,
                            int V, float* acc, void* out, bool first, bool last, bool accum,
                            hipStream_t s);

// Final loss: mean (sum / the row-weight sum in counts[2], NaN when 0) or
// sum, in float64, fixed order.
hipError_t loss_reduce(const float* loss_rows, int N, const int64_t* counts,
                       int reduction, float* loss, hipStream_t s);

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

// out[i] = in[i] * scale[(i / cols) * stride] for i < n (cols == 0: scale[0]
// everywhere), computed in fp32 and rounded to the element type; in == out
// allowed.  in and out 16-byte aligned; cols, when not 0, a multiple of the
// 16-byte vector width.
hipError_t scale(Elem e, const void* in, void* out, int64_t n, int64_t cols,
                 const float* scale, int64_t stride, hipStream_t s);

// Standalone CE: rows of fp32 logits overwritten with g_n (softmax - onehot);
// loss_rows[n] = w[n] (lse - z_t) (0 if tc < 0; w = wrow[n], 1 when null).
// z 4-byte aligned, any V >= 1.
hipError_t ce_inplace_rows(float* z, int N, int V, const int* tc, const float* g,
                           const float* wrow, float* loss_rows, hipStream_t s);

}  // namespace lce
