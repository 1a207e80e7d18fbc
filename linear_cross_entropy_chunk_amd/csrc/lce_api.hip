// C ABI of liblce.so: validation, chunk planning, workspace layout and the
// per-chunk launch sequence.  See include/lce.h for the contract.
//
// The chunk loop follows the batch-chunked accumulator of the PyTorch module
// torch/nn/modules/linear_cross_entropy.py: for each chunk of rows, the logits
// GEMM with bias, the row statistics and loss terms, then (when gradients are
// requested) the logits gradient in place and the three gradient products,
// with grad_W and grad_b accumulated across chunks in fp32 and committed to
// the input dtype once.  The chunk size defaults to the "aspect_ratio" rule of
// the torch.nn.LinearCrossEntropyOptions page.
#include "../../include/lce.h"
#include "lce_kernels.h"

#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

// Events bracketing selected kernel classes (the benchmark timing hook).
struct TimingPool {
  static constexpr size_t kPairs = 4096;
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev;   // 2 per slot
  std::vector<int> kind;        // kernel class per slot
  size_t used = 0;
  int64_t dropped = 0;          // launches of a timed class that found the pool full
};

struct lce_handle {
  lce_desc d;
  lce::Elem elem;     // element type of the inputs, gradients and T
  bool half;          // a 2-byte element type (bf16 or fp16): MFMA on 16-bit operands
  int esize;
  int64_t c;          // rows per chunk
  int64_t n_chunks;
  int64_t c_pad;      // c rounded up to 64 (row stride of dLt, Xt and partials)
  int64_t V_pad;      // V rounded up to 256 (row stride of T, Wt)
  int n_vt;           // statistics blocks of kStatCols classes
  int splits;         // split-K of the grad_X GEMM
  int k_split;
  int64_t grp;        // chunks per grad_W group (dL^T staged together)
  int64_t k_grp;      // columns of the dL^T / X^T staging buffers (grp * c_pad)
  int64_t n_groups;
  bool want_x, want_w, want_b, want_argmax, want_any;
  bool accum;         // add the gradients into the caller's buffers
  bool w_acc32;       // fp32 grad_W accumulator in the workspace
  bool w_inplace;     // grad_W reads dL where it lies in T (2-byte k-major operand)
  bool gx_group;      // one grad_X GEMM per grad_W group (its rows all in T)
  bool rowref;        // one reference per row: T holds dL / beta, no finalize pass
  bool grp_stats;     // chunks back to back in groups: statistics buffers for a whole
                      // group, so the combine (and the gated repair) can run per group
  int64_t ldp;        // row stride of the statistics partials and zt
  int64_t w_tail_cols;  // grad_W: trailing 256-class tile columns split along K (0: none)
  int w_tail_splits;    // K ranges of those columns
  int64_t gx_rows;    // most rows of one grad_X GEMM
  int64_t t_rows;     // rows R of the exp / dL buffer T (panel layout)
  // workspace offsets (bytes)
  size_t o_T, o_dLt, o_Wt, o_Xt, o_mp, o_sp, o_ip, o_zt, o_lse, o_g, o_tc, o_gxp,
      o_gw32, o_gbp, o_gb32, o_lrows, o_wrow, o_cnt, o_rref, o_beta, o_flag, o_wtail, total;
  TimingPool timing;
};

namespace {

thread_local char g_last_error[256] = "";

constexpr size_t kAlign = 256;
constexpr size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

lce_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LCE_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e),
           hipGetErrorString(e));
  return LCE_ERR_HIP;
}

#define LCE_HIP(call)                                  \
  do {                                                 \
    const lce_status st_ = hip_status(call);           \
    if (st_ != LCE_OK) return st_;                     \
  } while (0)

// Launch `call`; when the timing hook selects kernel class `k`, bracket it
// with two events on stream `s`.
#define LCE_LAUNCH(h, k, call)                                                   \
  do {                                                                           \
    TimingPool& tp_ = (h)->timing;                                               \
    const bool want_ = (tp_.mask >> (k)) & 1u;                                   \
    const bool on_ = want_ && tp_.used < tp_.kind.size();                        \
    if (want_ && !on_) ++tp_.dropped;                                            \
    if (on_) LCE_HIP(hipEventRecord(tp_.ev[2 * tp_.used], s));                   \
    LCE_HIP(call);                                                               \
    if (on_) {                                                                   \
      LCE_HIP(hipEventRecord(tp_.ev[2 * tp_.used + 1], s));                      \
      tp_.kind[tp_.used++] = (k);                                                \
    }                                                                            \
  } while (0)

// Fewest rows a logits launch covers when consecutive chunks can share one
// (eight 256-row tiles: each launch reads all of W once).
constexpr int64_t kLaunchRows = 2048;

// next power of two >= x (x >= 1)
int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Rows per chunk.  aspect_ratio: the logits buffer (rows, V) holds as many
// elements as the input (N, D): next_pow2(ceil(N / ceil(V / D))); the
// "aspect_ratio:N" form divides that by N (rounded down, at least 1 row).
int64_t resolve_chunk_rows(const lce_desc& d) {
  if (d.N == 0) return 0;
  int64_t c;
  if (d.chunk_rows > 0) c = d.chunk_rows;
  else if (d.chunk_rows == LCE_CHUNK_ALL) c = d.N;
  else c = std::max<int64_t>(1, next_pow2(cdiv64(d.N, cdiv64(d.V, d.D))) /
                                    std::max<int64_t>(1, d.chunk_divisor));
  return std::min(c, d.N);
}

void plan(lce_handle* h) {
  const lce_desc& d = h->d;
  h->elem = d.dtype == LCE_BF16 ? lce::Elem::kBF16
            : d.dtype == LCE_F16 ? lce::Elem::kF16 : lce::Elem::kF32;
  h->half = h->elem != lce::Elem::kF32;
  h->esize = lce::elem_size(h->elem);
  h->c = resolve_chunk_rows(d);
  h->n_chunks = h->c ? cdiv64(d.N, h->c) : 0;
  h->c_pad = round_up(std::max<int64_t>(h->c, 1), 64);
  h->V_pad = round_up(d.V, lce::kTile);
  h->n_vt = static_cast<int>(h->V_pad / lce::kStatCols);
  h->want_x = d.flags & LCE_GRAD_X;
  h->want_w = d.flags & LCE_GRAD_W;
  h->want_b = d.flags & LCE_GRAD_B;
  h->want_argmax = d.flags & LCE_ARGMAX;
  h->accum = d.flags & LCE_ACCUMULATE;
  h->want_any = h->want_x || h->want_w || h->want_b;

  // grad_W groups.  The dL of `grp` consecutive chunks stays in T (or is
  // staged as dL^T) and one GEMM with K = grp * c_pad rows forms their grad_W
  // contribution, so the accumulator is touched once per group instead of
  // once per chunk.  ACCURATE holds, by default, up to as many bytes of dL as
  // the fp32 V x D accumulator it saves (K up to 4 D / element size), or at
  // most group_rows rows when the descriptor sets it (group_rows <= the chunk
  // rows gives one chunk per group: each chunk's dL is consumed by both
  // gradient GEMMs right after it is formed, and grad_W is carried across
  // chunks in an fp32 accumulator).  COMPACT keeps one chunk per group (least
  // memory).  A non-mixed 16-bit layout (acc_dtype = the input dtype)
  // accumulates the gradients in the input dtype chunk by chunk: COMPACT's
  // grouping.
  const bool accurate = d.acc_policy == LCE_ACCURATE && !(h->half && d.acc_dtype == d.dtype);
  const int64_t k_max = d.group_rows > 0 ? d.group_rows : 4 * d.D / h->esize;
  h->grp = accurate ? std::max<int64_t>(1, k_max / h->c_pad) : 1;
  h->grp = std::max<int64_t>(1, std::min<int64_t>(h->grp, std::max<int64_t>(h->n_chunks, 1)));
  h->k_grp = h->grp * h->c_pad;
  h->n_groups = h->n_chunks ? cdiv64(h->n_chunks, h->grp) : 0;
  h->w_acc32 = h->want_w && h->half && accurate && h->n_groups > 1;
  // 2-byte types: the chunks of a group keep their dL in T (chunk j at row j c_pad of
  // every panel) and grad_W reads it there as a k-major operand, so dL^T is
  // not staged.  This needs the chunks back to back (c a multiple of 64, or
  // one chunk per group) so that T's rows line up with the staged X^T
  // columns.  Otherwise, and for fp32, the finalize stages dL^T.
  h->w_inplace = h->want_w && h->half && (h->c % 64 == 0 || h->grp == 1);
  h->t_rows = h->w_inplace ? h->k_grp : h->c_pad;

  // With the group's dL in T, grad_X runs once per group over all its rows
  // (fewer, larger launches; one split needs no partials and no split sum).
  h->gx_group = h->want_x && h->w_inplace;

  // One reference per row (bf16 gradients): the logits epilogue stores
  // exp(z - r_n) with r_n the row's target logit, so that
  // dL = beta_n (T with S_n taken off the target entry), beta_n = g_n / S_n.
  // beta then scales grad_X's columns in its epilogue, X^T's columns when it
  // is staged and T's rows in the grad_b column sums, and no pass rewrites T.
  // bf16 only: T's entries may exceed 1 (up to e^kRefGap), which fp16 cannot
  // hold.  Not with a staged dL^T, which the finalize pass forms.
  h->rowref = h->elem == lce::Elem::kBF16 && h->want_any && (!h->want_w || h->w_inplace);
  // With chunks of a multiple of 64 rows in groups of several, the chunks'
  // rows lie back to back in the statistics buffers, which hold a whole
  // group, so that the combine runs once per group instead of once per chunk
  // (fewer launches, and its rows span the group): for the one-reference
  // plan when the group's chunks all stay in T (with the gated repair, whose
  // flags cover the group's 256-row tiles, and the grad_b sums), and for
  // the loss-only forward of 'none'.
  h->grp_stats = h->grp > 1 && h->c % 64 == 0;

  // grad_W's last round.  D/256 x V/256 tiles on 256 CUs leave a partial
  // last round (at the large-vocabulary head 80 tiles: 31.3 rounds), during
  // which most CUs idle for a whole tile.  When that remainder is at most
  // half a round, the trailing V tile columns that hold it go to a second
  // launch with K split into ranges (fp32 partials, then the deterministic
  // split sum into grad_W's last rows), so the main launch ends on a full
  // round and the remainder takes a fraction of one.  Element-type store
  // modes only (no fp32 V x D accumulator).
  h->w_tail_cols = 0;
  h->w_tail_splits = 1;
  if (h->want_w && !h->w_acc32 && d.N > 0) {
    const int64_t tm = cdiv64(d.D, lce::kTile), tn = cdiv64(d.V, lce::kTile);
    const int64_t rem = (tm * tn) % 256;
    const int64_t cols = rem ? cdiv64(rem, tm) : 0;
    const int64_t k_max = h->grp * h->c_pad;                 // largest grad_W K
    if (cols > 0 && cols < tn && cols * tm <= 128) {
      // as many ranges as fill one round, each at least 4 stages deep
      const int64_t sp = std::min<int64_t>(256 / (cols * tm), k_max / 256);
      if (sp >= 2) {
        h->w_tail_cols = cols;
        h->w_tail_splits = static_cast<int>(sp);
      }
    }
  }
  h->gx_rows = h->gx_group ? std::min<int64_t>(h->grp * h->c, d.N) : h->c;
  // split-K for grad_X = dL . W: aim at one workgroup per CU (256; two
  // rounds of 512 measured slower: more partials to sum, twice the tile
  // starts), >= 64 K per split (one stage; a small problem would otherwise
  // leave a few workgroups walking all of K through mostly empty 256 x 256
  // tiles).
  const int64_t tiles = cdiv64(h->gx_rows, lce::kTile) * cdiv64(d.D, lce::kTile);
  int64_t splits = std::max<int64_t>(1, cdiv64(256, std::max<int64_t>(tiles, 1)));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, h->V_pad / 64));
  int64_t ks = round_up(cdiv64(h->V_pad, splits), 64);
  h->splits = static_cast<int>(cdiv64(h->V_pad, ks));
  h->k_split = static_cast<int>(ks);

  const int64_t es = h->esize, c = h->c_pad, V = d.V, Vp = h->V_pad, D = d.D, N = d.N;
  size_t o = 0;
  auto take = [&](size_t bytes, bool need) {
    const size_t at = o;
    if (need) o = align_up(o + bytes);
    return need ? at : static_cast<size_t>(-1);
  };
  h->o_T = take(h->t_rows * Vp * es, h->want_any);
  h->o_dLt = take(Vp * h->k_grp * es, h->want_w && !h->w_inplace);
  // 2-byte grad_X reads W in place (k-major operand); fp32 uses a transposed copy
  h->o_Wt = take(D * Vp * es, h->want_x && !h->half);
  h->o_Xt = take(D * h->k_grp * es, h->want_w);
  h->ldp = h->grp_stats ? h->k_grp : c;
  h->o_mp = take(h->n_vt * h->ldp * 4, true);
  h->o_sp = take(h->n_vt * h->ldp * 4, true);
  h->o_ip = take(h->n_vt * h->ldp * 4, h->want_argmax);
  h->o_zt = take(h->ldp * 4, true);
  h->o_lse = take(h->ldp * 4, true);
  h->o_g = take(std::max<int64_t>(N, 1) * 4, true);
  h->o_tc = take(std::max<int64_t>(N, 1) * 4, true);
  h->o_gxp = take(static_cast<size_t>(h->splits) * round_up(h->gx_rows, 64) * D * 4,
                  h->want_x && !(h->gx_group && h->splits == 1));
  h->o_gw32 = take(V * D * 4, h->w_acc32);
  // the finalize's grad_b partials, one row per 64 rows it covers: a whole
  // group when short chunks share their logits launch (16-bit gradients,
  // finalize per group)
  const bool fin_group = h->grp_stats && h->c < kLaunchRows && h->w_inplace;
  h->o_gbp = take(((fin_group ? h->k_grp : c) / 64) * Vp * 4, h->want_b && !h->rowref);
  h->o_gb32 = take(Vp * 4, h->want_b);
  h->o_lrows = take(std::max<int64_t>(N, 1) * 4, true);
  h->o_wrow = take(std::max<int64_t>(N, 1) * 4, true);
  // n_valid, n_bad, row-weight sum (double), then the fp16 dL scale 2^k and 2^-k
  h->o_cnt = take(3 * 8 + 2 * 4, true);
  h->o_rref = take(std::max<int64_t>(N, 1) * 4, h->rowref);
  h->o_beta = take(std::max<int64_t>(N, 1) * 4, h->rowref);
  // one repair flag per 256-row tile of each chunk (chunk ck's at ck * fpc)
  h->o_flag = take(std::max<int64_t>(h->n_chunks * cdiv64(h->c_pad, lce::kTile), 1) * 4,
                   h->rowref);
  h->o_wtail = take(static_cast<size_t>(h->w_tail_splits) * h->w_tail_cols * lce::kTile * D * 4,
                    h->w_tail_cols > 0);
  h->total = o;
}

template <typename T>
T* at(void* ws, size_t off) {
  return off == static_cast<size_t>(-1) ? nullptr
                                         : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Scratch of the standalone CE on N rows: corrected targets, row weights g,
// per-row losses and class weights (N each, 4 bytes), then the counters
// (n_valid, n_bad, the weight sum).
size_t ce_scratch_bytes(int64_t N) {
  const int64_t n = std::max<int64_t>(N, 1);
  return align_up(n * 4) * 4 + align_up(24);
}

// Host validation shared by both CE entry points.
lce_status ce_check(const float* logits, const int64_t* targets, int64_t N, int64_t V,
                    int32_t reduction, const float* loss) {
  if (N < 0 || V < 1) return LCE_ERR_INVALID_ARG;
  if (reduction < LCE_MEAN || reduction > LCE_NONE) return LCE_ERR_UNSUPPORTED;
  if (N > 0 && (!logits || !targets)) return LCE_ERR_INVALID_ARG;
  if (!loss) return LCE_ERR_INVALID_ARG;
  if (logits && (reinterpret_cast<uintptr_t>(logits) & 3) != 0) return LCE_ERR_UNSUPPORTED;
  if (N > 2147483647LL || V > 2147483647LL) return LCE_ERR_UNSUPPORTED;
  return LCE_OK;
}

// The standalone CE's launches on scratch `ws` (ce_scratch_bytes(N) bytes):
// target prep (row weights, counts), the in-place rows, the loss reduction.
// Every scratch element a launch reads was written by an earlier launch of
// the same call, so the scratch needs no clearing.
lce_status ce_enqueue(float* logits, const int64_t* targets, const float* class_weight,
                      int64_t N, int64_t V, int64_t ignore_index, int32_t reduction,
                      float grad_scale, float* loss, int64_t* n_valid, char* ws,
                      hipStream_t s) {
  const int64_t n = std::max<int64_t>(N, 1);
  int* tc = reinterpret_cast<int*>(ws);
  float* g = reinterpret_cast<float*>(ws + align_up(n * 4));
  float* lrows = reinterpret_cast<float*>(ws + 2 * align_up(n * 4));
  float* wrow = reinterpret_cast<float*>(ws + 3 * align_up(n * 4));
  int64_t* cnt = reinterpret_cast<int64_t*>(ws + 4 * align_up(n * 4));
  const bool none = reduction == LCE_NONE;
  // Per-row weights: 'none' takes grad_scale on every counted row, which is
  // the weight the 'sum' reduction gives.
  LCE_HIP(lce::prep_targets(targets, static_cast<int>(N), static_cast<int>(V), ignore_index,
                            none ? LCE_SUM : reduction, grad_scale, nullptr, class_weight, tc, g,
                            wrow, cnt, n_valid, nullptr, nullptr, s));
  LCE_HIP(lce::ce_inplace_rows(logits, static_cast<int>(N), static_cast<int>(V), tc, g,
                               class_weight ? wrow : nullptr, none ? loss : lrows, s));
  if (!none) LCE_HIP(lce::loss_reduce(lrows, static_cast<int>(N), cnt, reduction, loss, s));
  return LCE_OK;
}

// The allocation-free CE's scratch: one static array per device, sized for
// LCE_CE_NOALLOC_MAX_ROWS rows.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes =
    (LCE_CE_NOALLOC_MAX_ROWS * 4 + kAlign - 1) / kAlign * kAlign * 4 + kAlign;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call there.
lce_status noalloc_scratch(char** out) {
  int dev = 0;
  LCE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return LCE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    LCE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return LCE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return LCE_OK;
}
static_assert(kNoAllocScratchBytes >= align_up(LCE_CE_NOALLOC_MAX_ROWS * 4) * 4 + align_up(24),
              "the static scratch holds ce_scratch_bytes(LCE_CE_NOALLOC_MAX_ROWS)");

}  // namespace

extern "C" {

const char* lce_status_string(lce_status s) {
  // A caller may pass any int (C, or the Python binding); a C++ load of an
  // lce_status outside its enumerators is undefined, so read the bits.
  int code = 0;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case LCE_OK: return "LCE_OK";
    case LCE_ERR_INVALID_ARG: return "LCE_ERR_INVALID_ARG";
    case LCE_ERR_DTYPE: return "LCE_ERR_DTYPE";
    case LCE_ERR_UNSUPPORTED: return "LCE_ERR_UNSUPPORTED";
    case LCE_ERR_WORKSPACE: return "LCE_ERR_WORKSPACE";
    case LCE_ERR_HIP: return "LCE_ERR_HIP";
  }
  return "LCE_ERR_UNKNOWN";
}

const char* lce_last_error(void) { return g_last_error; }

lce_status lce_create(const lce_desc* d, lce_handle** out) {
  if (!d || !out) return LCE_ERR_INVALID_ARG;
  *out = nullptr;
  if (d->N < 0 || d->D < 1 || d->V < 1 || d->chunk_rows < LCE_CHUNK_ALL ||
      d->chunk_divisor < 0 || d->group_rows < 0)
    return LCE_ERR_INVALID_ARG;
  if (d->dtype != LCE_F32 && d->dtype != LCE_BF16 && d->dtype != LCE_F16) return LCE_ERR_DTYPE;
  // an unknown reduction is the pages' NotImplementedError
  if (d->reduction < LCE_MEAN || d->reduction > LCE_NONE) return LCE_ERR_UNSUPPORTED;
  if (d->acc_policy != LCE_ACCURATE && d->acc_policy != LCE_COMPACT) return LCE_ERR_INVALID_ARG;
  if (d->has_bias != 0 && d->has_bias != 1) return LCE_ERR_INVALID_ARG;
  if (d->flags &
      ~static_cast<uint32_t>(LCE_GRAD_X | LCE_GRAD_W | LCE_GRAD_B | LCE_ARGMAX | LCE_ACCUMULATE))
    return LCE_ERR_INVALID_ARG;
  if ((d->flags & LCE_GRAD_B) && !d->has_bias) return LCE_ERR_INVALID_ARG;
  // Mixed precision is bf16 / fp16 (or fp32) inputs with an fp32 accumulator;
  // an accumulator of the input dtype itself is the non-mixed layout.
  if (d->acc_dtype != LCE_F32 && d->acc_dtype != d->dtype) return LCE_ERR_UNSUPPORTED;
  const int64_t vec = d->dtype == LCE_F32 ? 4 : 8;
  if (d->D % vec != 0) return LCE_ERR_UNSUPPORTED;
  const int64_t kMax = 2147483647LL - 1024;
  if (d->N > kMax || d->V > kMax || d->D > kMax) return LCE_ERR_UNSUPPORTED;
  // The GEMMs address the rows of a 256-row operand tile with 32-bit byte
  // offsets, so each operand's row length (D; the chunk and group rows for
  // the staged X^T / dL^T; V_pad for fp32's W^T) times 256 rows must stay
  // below 2 GiB.  These limits keep every one at or below 1 GiB.
  constexpr int64_t kMaxRowLen = int64_t{1} << 20;
  if (d->D > kMaxRowLen) return LCE_ERR_UNSUPPORTED;
  lce_handle* h = new (std::nothrow) lce_handle();
  if (!h) return LCE_ERR_INVALID_ARG;
  h->d = *d;
  plan(h);
  if (h->c > kMaxRowLen || (!h->half && h->want_x && h->V_pad >= 2 * kMaxRowLen)) {
    delete h;
    return LCE_ERR_UNSUPPORTED;
  }
  *out = h;
  return LCE_OK;
}

lce_status lce_workspace_size(const lce_handle* h, size_t* bytes) {
  if (!h || !bytes) return LCE_ERR_INVALID_ARG;
  *bytes = h->total;
  return LCE_OK;
}

lce_status lce_chunk_info(const lce_handle* h, int64_t* chunk_rows, int64_t* n_chunks) {
  if (!h) return LCE_ERR_INVALID_ARG;
  if (chunk_rows) *chunk_rows = h->c;
  if (n_chunks) *n_chunks = h->n_chunks;
  return LCE_OK;
}

lce_status lce_timing_enable(lce_handle* h, uint32_t kernel_mask) {
  if (!h) return LCE_ERR_INVALID_ARG;
  TimingPool& tp = h->timing;
  if (kernel_mask == 0) {
    for (hipEvent_t e : tp.ev) (void)hipEventDestroy(e);
    tp.ev.clear();
    tp.kind.clear();
    tp.used = 0;
    tp.dropped = 0;
    tp.mask = 0;
    return LCE_OK;
  }
  if (tp.ev.empty()) {
    tp.ev.resize(2 * TimingPool::kPairs, nullptr);
    for (hipEvent_t& e : tp.ev) LCE_HIP(hipEventCreate(&e));
    tp.kind.assign(TimingPool::kPairs, 0);
  }
  tp.used = 0;
  tp.dropped = 0;
  tp.mask = kernel_mask;
  return LCE_OK;
}

lce_status lce_timing_read(lce_handle* h, double* ms, int64_t* launches) {
  if (!h) return LCE_ERR_INVALID_ARG;
  TimingPool& tp = h->timing;
  double tot[LCE_K_COUNT] = {0};
  int64_t cnt[LCE_K_COUNT] = {0};
  if (tp.used > 0) LCE_HIP(hipEventSynchronize(tp.ev[2 * tp.used - 1]));
  for (size_t i = 0; i < tp.used; ++i) {
    float t = 0.0f;
    LCE_HIP(hipEventElapsedTime(&t, tp.ev[2 * i], tp.ev[2 * i + 1]));
    tot[tp.kind[i]] += t;
    cnt[tp.kind[i]] += 1;
  }
  tp.used = 0;
  for (int k = 0; k < LCE_K_COUNT; ++k) {
    if (ms) ms[k] = tot[k];
    if (launches) launches[k] = cnt[k];
  }
  if (tp.dropped > 0) {
    // the totals cover the timed launches only: say so rather than let a
    // partial count pass for a whole one
    snprintf(g_last_error, sizeof(g_last_error),
             "lce_timing_read: %lld launches found the pool of %zu event pairs full and "
             "were not timed", static_cast<long long>(tp.dropped), TimingPool::kPairs);
    tp.dropped = 0;
    return LCE_ERR_UNSUPPORTED;
  }
  return LCE_OK;
}

lce_status lce_destroy(lce_handle* h) {
  if (h) lce_timing_enable(h, 0);
  delete h;
  return LCE_OK;
}

lce_status lce_forward_backward(lce_handle* h, const lce_io* io, void* workspace, size_t ws_bytes,
                                void* stream) {
  if (!h || !io) return LCE_ERR_INVALID_ARG;
  const lce_desc& d = h->d;
  const bool none = d.reduction == LCE_NONE;
  if (!none && io->grad_output) return LCE_ERR_INVALID_ARG;
  const bool grads = h->want_any && (!none || io->grad_output != nullptr);
  const bool want_x = grads && h->want_x, want_w = grads && h->want_w,
             want_b = grads && h->want_b;
  if (!io->targets && d.N > 0) return LCE_ERR_INVALID_ARG;
  if (d.N > 0 && (!io->X || !io->W)) return LCE_ERR_INVALID_ARG;
  if (d.has_bias && !io->b) return LCE_ERR_INVALID_ARG;
  if (!d.has_bias && io->b) return LCE_ERR_INVALID_ARG;
  if (!io->loss && !(none && io->grad_output)) return LCE_ERR_INVALID_ARG;
  if ((want_x && !io->grad_X && d.N > 0) || (want_w && !io->grad_W) || (want_b && !io->grad_b))
    return LCE_ERR_INVALID_ARG;
  if (h->want_argmax && !io->argmax && d.N > 0) return LCE_ERR_INVALID_ARG;
  if ((io->X && !aligned16(io->X)) || (io->W && !aligned16(io->W)))
    return LCE_ERR_UNSUPPORTED;
  if (h->total > 0 && (!workspace || ws_bytes < h->total ||
                       (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))))
    return LCE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const lce::Elem el = h->elem;
  const bool half = h->half;
  const int es = h->esize;
  const int N = static_cast<int>(d.N), D = static_cast<int>(d.D), V = static_cast<int>(d.V);
  const int64_t cp = h->c_pad, Vp = h->V_pad;
  void* T = at<char>(workspace, h->o_T);
  void* dLt = at<char>(workspace, h->o_dLt);
  void* Wt = at<char>(workspace, h->o_Wt);
  void* Xt = at<char>(workspace, h->o_Xt);
  float* mp = at<float>(workspace, h->o_mp);
  float* sp = at<float>(workspace, h->o_sp);
  int* ip = at<int>(workspace, h->o_ip);
  float* zt = at<float>(workspace, h->o_zt);
  float* lse = at<float>(workspace, h->o_lse);
  float* g = at<float>(workspace, h->o_g);
  int* tc = at<int>(workspace, h->o_tc);
  float* gxp = at<float>(workspace, h->o_gxp);
  float* gw32 = at<float>(workspace, h->o_gw32);
  float* gbp = at<float>(workspace, h->o_gbp);
  float* gb32 = at<float>(workspace, h->o_gb32);
  float* lrows = at<float>(workspace, h->o_lrows);
  float* wrow = at<float>(workspace, h->o_wrow);
  int64_t* cnt = at<int64_t>(workspace, h->o_cnt);
  const bool rowref = h->rowref && grads;
  // the combine per group (statistics of the whole group): the one-reference
  // plan with the group's chunks in T, or a call without gradients
  const bool grp_comb = h->grp_stats && (rowref ? h->w_inplace : !grads);
  // Short chunks make poor logits launches: below 256 rows most rows of
  // every tile are empty, and each launch reads all of W again, so 256-row
  // chunks read it eight times as often as 2048-row ones.  When a group's
  // chunks lie back to back in T and in group-sized statistics (the combine
  // per group, or 16-bit gradients), consecutive chunks share a logits launch
  // of at least kLaunchRows rows (at most the group), which writes the layout
  // the chunks' own launches would.  Chunks of kLaunchRows or more keep one
  // launch each.
  const bool share_ok = h->grp_stats && (grp_comb || (grads && h->w_inplace));
  const int64_t unit = share_ok ? std::max<int64_t>(1, cdiv64(kLaunchRows, h->c)) : 1;
  const bool merge = unit > 1;
  float* rref = at<float>(workspace, h->o_rref);
  float* beta = at<float>(workspace, h->o_beta);
  // repair flags, one per 256-row tile of a chunk, so that a row whose
  // reference is too low costs the recompute of its tile's rows only
  int* flags = at<int>(workspace, h->o_flag);
  const int64_t fpc = cdiv64(h->c_pad, lce::kTile);
  // fp16 keeps dL times a power of two 2^k (from the largest row weight) so
  // that it stays inside fp16's range; the gradients' element-type stores
  // multiply by 2^-k.  Exact scalings: no rounding is added.
  float* dl_scale = h->elem == lce::Elem::kF16 ? reinterpret_cast<float*>(cnt + 3) : nullptr;
  const float* dl_unscale = dl_scale ? dl_scale + 1 : nullptr;

  LCE_LAUNCH(h, LCE_K_PREP, lce::prep_targets(io->targets, N, V, d.ignore_index, d.reduction, io->grad_scale,
                            io->grad_output, io->class_weight, tc, g, wrow, cnt, io->n_valid,
                            io->n_bad, dl_scale, s));

  if (N == 0) {
    if (want_w && !h->accum) LCE_LAUNCH(h, LCE_K_LOSS, lce::fill_zero(io->grad_W, static_cast<size_t>(d.V) * d.D * es, s));
    if (want_b && !h->accum) LCE_LAUNCH(h, LCE_K_LOSS, lce::fill_zero(io->grad_b, static_cast<size_t>(d.V) * es, s));
    if (!none) LCE_LAUNCH(h, LCE_K_LOSS, lce::loss_reduce(lrows, 0, cnt, d.reduction, io->loss, s));
    return LCE_OK;
  }

  if (want_x && !half)
    LCE_LAUNCH(h, LCE_K_TRANSPOSE, lce::transpose_pad(el, io->W, D, V, D, Wt, Vp, static_cast<int>(Vp), s));
  if (rowref)
    LCE_LAUNCH(h, LCE_K_PREP, lce::target_logits(el, io->X, D, io->W, D, io->b, tc, N, D, rref,
                                                 flags, static_cast<int>(h->n_chunks * fpc), s));

  // grad_X[xrow0 .. + nrows) = dL . W for dL rows held in T from Tb on, with
  // M = D against dL[rows][V] (K = V): the transposed store writes grad_X
  // rows with contiguous vectors.  2-byte types read W[V][D] itself as a
  // k-major operand (rows past V read as 0); fp32 reads the transposed copy
  // W^T[D][V_pad].  With one split (2-byte types) the GEMM writes grad_X
  // itself; otherwise fp32 split partials are summed into it.
  auto grad_x = [&](void* Tb, int64_t xrow0, int nrows) -> lce_status {
    const int64_t tps = h->t_rows * lce::kTile;
    lce::GemmNT gx{};
    if (half) {
      gx.A = io->W; gx.lda = D; gx.a_kmajor = true; gx.a_krows = V;
    } else {
      gx.A = Wt; gx.lda = Vp;
    }
    gx.B = Tb; gx.ldb = lce::kTile; gx.b_pstride = tps;
    gx.M = D; gx.N = nrows; gx.K = static_cast<int>(Vp);
    gx.splits = h->splits; gx.k_split = h->k_split;
    gx.split_stride = static_cast<int64_t>(nrows) * D;
    gx.ldc = D; gx.Cin = nullptr;
    gx.group_m = 4;   // an XCD's 32 concurrent tiles: 4 along D x 8 along rows
    gx.role = lce::GemmRole::kGradX;
    char* out = static_cast<char*>(io->grad_X) + xrow0 * d.D * es;
    // one-reference plan: grad_X row n = beta_n (T . W)[n]
    const float* rs = rowref ? beta + xrow0 : nullptr;
    if (half && h->splits == 1) {
      gx.C = out;
      gx.mode = h->accum ? lce::EpiMode::kAccumOut : lce::EpiMode::kStoreOut;
      gx.out_scale = dl_unscale;
      gx.n_scale = rs;
      LCE_LAUNCH(h, LCE_K_GEMM_X, lce::gemm_nt(el, gx, s));
      return LCE_OK;
    }
    gx.C = gxp;
    gx.mode = lce::EpiMode::kStoreF32;
    LCE_LAUNCH(h, LCE_K_GEMM_X, lce::gemm_nt(el, gx, s));
    LCE_LAUNCH(h, LCE_K_SPLIT_SUM, lce::sum_splits(el, gxp, h->splits, gx.split_stride, nrows, D,
                                                   out, h->accum, dl_unscale, s, rs));
    return LCE_OK;
  };

  const char* Xb = static_cast<const char*>(io->X);
  for (int64_t ck = 0; ck < h->n_chunks; ++ck) {
    const int64_t row0 = ck * h->c;
    const int rows = static_cast<int>(std::min<int64_t>(h->c, d.N - row0));
    const int rows_pad = static_cast<int>(round_up(rows, 64));
    const bool first = ck == 0, last = ck + 1 == h->n_chunks;
    const void* Xc = Xb + row0 * d.D * es;
    const int64_t jj = ck % h->grp;               // position inside the grad_W group
    const int64_t tps = h->t_rows * lce::kTile;   // T's panel stride (elements)
    void* Tc = static_cast<char*>(T) + (h->w_inplace ? jj * cp : 0) * lce::kTile * es;

    lce::LogitsLse la{};
    la.X = Xc; la.ldx = D;
    la.W = io->W; la.ldw = D;
    la.bias = io->b;
    la.tc = tc + row0;
    la.rows = rows; la.V = V; la.D = D;
    la.T = grads ? Tc : nullptr; la.tps = tps;
    // statistics of the chunk's rows: at column jj c_pad of the group's
    // buffers when the combine runs per group or the launch is shared, else
    // at column 0
    const int64_t sc = (grp_comb || merge) ? jj * cp : 0;
    la.m_part = mp + sc; la.s_part = sp + sc;
    la.i_part = h->want_argmax ? ip + sc : nullptr; la.ldp = h->ldp;
    la.zt = zt + sc;
    // one-reference plan: the padding rows up to rows_pad are written as 0
    // (grad_W's K range covers them)
    la.rref = rowref ? rref + row0 : nullptr;
    la.t_rows = rowref ? rows_pad : rows;
    la.gate = nullptr;
    if (!merge) {
      LCE_LAUNCH(h, LCE_K_LOGITS, lce::logits_lse(el, la, s));
    } else if (jj % unit == 0) {
      // this chunk and the next unit - 1 of its group
      const int64_t u_rows =
          std::min<int64_t>(std::min(unit, h->grp - jj) * h->c, d.N - row0);
      la.rows = static_cast<int>(u_rows);
      la.t_rows = static_cast<int>(rowref ? round_up(u_rows, 64) : u_rows);
      LCE_LAUNCH(h, LCE_K_LOGITS, lce::logits_lse(el, la, s));
    }

    float* loss_rows = (none && io->loss) ? io->loss + row0 : lrows + row0;
    const float* wrow_c = io->class_weight ? wrow + row0 : nullptr;
    int* amax_c = h->want_argmax ? io->argmax + row0 : nullptr;
    // combine, then the repair of rows whose reference was too low: both
    // repair launches do nothing unless the combine raised a flag.  Per
    // chunk here, or per group at the group's end (below).
    auto combine_ref = [&](lce::LogitsLse lr, int64_t r0, int nrows, void* Tb, int* flag,
                           int flag_rows) -> lce_status {
      float* loss_r = (none && io->loss) ? io->loss + r0 : lrows + r0;
      const float* wrow_r = io->class_weight ? wrow + r0 : nullptr;
      int* amax_r = h->want_argmax ? io->argmax + r0 : nullptr;
      LCE_LAUNCH(h, LCE_K_COMBINE,
                 lce::row_combine_ref(lr.m_part, lr.s_part, lr.i_part, h->ldp, h->n_vt, lr.zt,
                                      tc + r0, wrow_r, g + r0, nrows, rref + r0, Tb, tps, loss_r,
                                      beta + r0, amax_r, flag, flag_rows, nullptr, s));
      lr.gate = flag;
      lr.gate_rows = flag_rows;
      LCE_LAUNCH(h, LCE_K_REPAIR, lce::logits_lse(el, lr, s));
      LCE_LAUNCH(h, LCE_K_REPAIR,
                 lce::row_combine_ref(lr.m_part, lr.s_part, lr.i_part, h->ldp, h->n_vt, lr.zt,
                                      tc + r0, wrow_r, g + r0, nrows, rref + r0, Tb, tps, loss_r,
                                      beta + r0, amax_r, flag, flag_rows, flag, s));
      return LCE_OK;
    };
    if (rowref && !grp_comb) {
      const lce_status st = combine_ref(la, row0, rows, Tc, flags + ck * fpc, lce::kTile);
      if (st != LCE_OK) return st;
    } else if (rowref) {
      // per group: the group's last chunk runs it below
    } else if (grp_comb) {
      // no gradients (the loss-only forward of 'none', or a call that asks
      // for none): the group's combine after its last chunk's logits
      if (jj + 1 == h->grp || last) {
        const int64_t g_row0 = (ck - jj) * h->c;
        const int g_rows = static_cast<int>(row0 + rows - g_row0);
        float* loss_g = (none && io->loss) ? io->loss + g_row0 : lrows + g_row0;
        LCE_LAUNCH(h, LCE_K_COMBINE,
                   lce::row_combine(mp, sp, ip, h->ldp, h->n_vt, zt, tc + g_row0,
                                    io->class_weight ? wrow + g_row0 : nullptr, g_rows, lse,
                                    loss_g, h->want_argmax ? io->argmax + g_row0 : nullptr, s));
      }
      continue;
    } else if (merge) {
      // 16-bit gradients whose chunks shared a logits launch: the combine,
      // the finalize and the grad_b partials once per group, over the
      // group's rows back to back in T, after its last chunk
      if (jj + 1 == h->grp || last) {
        const int64_t g_row0 = (ck - jj) * h->c;
        const int g_rows = static_cast<int>(row0 + rows - g_row0);
        const int g_rows_pad = static_cast<int>(round_up(g_rows, 64));
        float* loss_g = (none && io->loss) ? io->loss + g_row0 : lrows + g_row0;
        LCE_LAUNCH(h, LCE_K_COMBINE,
                   lce::row_combine(mp, sp, ip, h->ldp, h->n_vt, zt, tc + g_row0,
                                    io->class_weight ? wrow + g_row0 : nullptr, g_rows, lse,
                                    loss_g, h->want_argmax ? io->argmax + g_row0 : nullptr, s));
        LCE_LAUNCH(h, LCE_K_FINALIZE,
                   lce::finalize_dlogits(el, T, tps, nullptr, h->k_grp, mp, h->ldp, lse,
                                         g + g_row0, tc + g_row0, g_rows, g_rows_pad, V,
                                         static_cast<int>(Vp), want_b ? gbp : nullptr, dl_scale,
                                         s));
        if (want_b)
          LCE_LAUNCH(h, LCE_K_BIAS, lce::bias_grad_reduce(el, gbp, g_rows_pad / 64, Vp, V, gb32,
                                                          io->grad_b, ck - jj == 0, last,
                                                          h->accum, s));
      }
    } else {
      LCE_LAUNCH(h, LCE_K_COMBINE, lce::row_combine(mp, sp, ip, h->ldp, h->n_vt, zt, tc + row0,
                                                    wrow_c, rows, lse, loss_rows, amax_c, s));
      if (!grads) continue;
      char* dLt_j = dLt ? static_cast<char*>(dLt) + jj * cp * es : nullptr;
      LCE_LAUNCH(h, LCE_K_FINALIZE, lce::finalize_dlogits(el, Tc, tps,
                                    want_w && !h->w_inplace ? dLt_j : nullptr,
                                    h->k_grp, mp, h->ldp, lse, g + row0, tc + row0, rows, rows_pad,
                                    V, static_cast<int>(Vp), want_b ? gbp : nullptr, dl_scale, s));
    }
    if (want_x && !h->gx_group) {
      const lce_status st = grad_x(Tc, row0, rows);
      if (st != LCE_OK) return st;
    }
    if (want_w) {
      // X^T of the group for grad_W: per chunk when dL^T is staged, else once
      // for the whole group at its end (its rows back to back, as in T)
      if (!h->w_inplace)
        LCE_LAUNCH(h, LCE_K_TRANSPOSE, lce::transpose_pad(el, Xc, D, rows, D,
                                                          static_cast<char*>(Xt) + jj * cp * es,
                                                          h->k_grp, rows_pad, s));
      if (jj + 1 == h->grp || last) {
        const int64_t g_row0 = (ck - jj) * h->c;
        const int g_rows = static_cast<int>(row0 + rows - g_row0);
        const int64_t gi = ck / h->grp;
        const bool gfirst = gi == 0, glast = last;
        if (rowref && grp_comb) {
          // the group's rows back to back from T's row 0 and statistics
          // column 0; one flag per 256-row tile
          lce::LogitsLse lg = la;
          lg.X = Xb + g_row0 * d.D * es;
          lg.tc = tc + g_row0;
          lg.rows = g_rows;
          lg.T = T;
          lg.m_part = mp; lg.s_part = sp; lg.i_part = h->want_argmax ? ip : nullptr;
          lg.zt = zt;
          lg.rref = rref + g_row0;
          lg.t_rows = static_cast<int>(round_up(g_rows, 64));
          // (flags by 256-row tile of the group, from its first chunk's
          // first flag: cdiv(g_rows, 256) of them, within the grp * fpc
          // flags its chunks own, since every chunk owns at least one)
          const lce_status st = combine_ref(lg, g_row0, g_rows, T, flags + (ck - jj) * fpc,
                                            lce::kTile);
          if (st != LCE_OK) return st;
          if (want_b)
            LCE_LAUNCH(h, LCE_K_BIAS, lce::bias_cols(T, tps, beta + g_row0, g_rows, V, gb32,
                                                     io->grad_b, gfirst, glast, h->accum, s));
        }
        // (one-reference plan: X^T's column k times beta_k)
        if (h->w_inplace)
          LCE_LAUNCH(h, LCE_K_TRANSPOSE, lce::transpose_pad(el, Xb + g_row0 * d.D * es, D, g_rows,
                                                            D, Xt, h->k_grp,
                                                            static_cast<int>(round_up(g_rows, 64)),
                                                            s, rowref ? beta + g_row0 : nullptr));
        if (want_x && h->gx_group) {
          // the whole group's rows, back to back in T from row 0
          const lce_status st = grad_x(T, g_row0, g_rows);
          if (st != LCE_OK) return st;
        }
        // grad_W[V][D] += dL^T . X over the group's rows, as (X^T)[D][K]
        // against dL^T with the transposed store: in place, dL is T's panels
        // read k-major; staged, the finalize's dL^T[V][K].
        lce::GemmNT gw{};
        gw.A = Xt; gw.lda = h->k_grp;
        gw.K = static_cast<int>(jj * cp + rows_pad);
        if (h->w_inplace) {
          gw.B = T; gw.ldb = lce::kTile; gw.b_pstride = tps;
          gw.b_kmajor = true; gw.b_krows = gw.K;
        } else {
          gw.B = dLt; gw.ldb = h->k_grp;
        }
        gw.M = D; gw.N = V;
        gw.splits = 1; gw.k_split = gw.K; gw.split_stride = 0;
        gw.ldc = D;
        gw.group_m = 4;   // an XCD's 32 concurrent tiles: 4 along D x 8 along V
        gw.role = lce::GemmRole::kGradW;
        if (h->w_acc32) {
          if (gfirst) { gw.C = gw32; gw.mode = lce::EpiMode::kStoreF32; }
          else if (!glast) { gw.C = gw32; gw.mode = lce::EpiMode::kAccumF32; }
          else {
            gw.C = io->grad_W; gw.Cin = gw32;
            gw.mode = h->accum ? lce::EpiMode::kFinalAccum : lce::EpiMode::kFinalOut;
          }
        } else {
          gw.C = io->grad_W;
          gw.mode = gfirst && !h->accum ? lce::EpiMode::kStoreOut : lce::EpiMode::kAccumOut;
        }
        gw.out_scale = dl_unscale;
        // the trailing tile columns of a partial last round, split along K:
        // classes from the first of those columns on (a tile boundary, also
        // when the last column is ragged)
        const int64_t v_main =
            std::max<int64_t>(0, cdiv64(V, lce::kTile) - h->w_tail_cols) * lce::kTile;
        const int k_split = static_cast<int>(   // whole 64-deep stages for every element type
            round_up(cdiv64(gw.K, std::max(h->w_tail_splits, 1)), 64));
        const int t_splits = static_cast<int>(cdiv64(gw.K, k_split));
        if (h->w_tail_cols > 0 && t_splits >= 2 && v_main > 0) {
          lce::GemmNT gt = gw;
          gw.N = static_cast<int>(v_main);
          gt.N = static_cast<int>(V - v_main);
          if (h->w_inplace) gt.B = static_cast<const char*>(gw.B) + (v_main / lce::kTile) * tps * es;
          else gt.B = static_cast<const char*>(gw.B) + v_main * h->k_grp * es;
          gt.splits = t_splits;
          gt.k_split = k_split;
          gt.split_stride = static_cast<int64_t>(gt.N) * D;
          gt.C = at<float>(workspace, h->o_wtail);
          gt.mode = lce::EpiMode::kStoreF32;
          gt.out_scale = nullptr;
          LCE_LAUNCH(h, LCE_K_GEMM_W, lce::gemm_nt(el, gw, s));
          LCE_LAUNCH(h, LCE_K_GEMM_W, lce::gemm_nt(el, gt, s));
          LCE_LAUNCH(h, LCE_K_SPLIT_SUM,
                     lce::sum_splits(el, static_cast<const float*>(gt.C), t_splits,
                                     gt.split_stride, gt.N, D,
                                     static_cast<char*>(io->grad_W) + v_main * D * es,
                                     gw.mode == lce::EpiMode::kAccumOut, dl_unscale, s));
        } else {
          LCE_LAUNCH(h, LCE_K_GEMM_W, lce::gemm_nt(el, gw, s));
        }
      }
    }
    if (want_b && rowref && !grp_comb)
      LCE_LAUNCH(h, LCE_K_BIAS, lce::bias_cols(Tc, tps, beta + row0, rows, V, gb32, io->grad_b,
                                               first, last, h->accum, s));
    else if (want_b && !rowref && !merge)
      LCE_LAUNCH(h, LCE_K_BIAS, lce::bias_grad_reduce(el, gbp, rows_pad / 64, Vp, V, gb32, io->grad_b, first,
                                    last, h->accum, s));
  }
  if (!none) LCE_LAUNCH(h, LCE_K_LOSS, lce::loss_reduce(lrows, N, cnt, d.reduction, io->loss, s));
  return LCE_OK;
}

lce_status lce_ce_workspace_size(int64_t N, int64_t V, size_t* bytes) {
  if (!bytes || N < 0 || V < 1) return LCE_ERR_INVALID_ARG;
  *bytes = ce_scratch_bytes(N);
  return LCE_OK;
}

lce_status lce_scale(const void* in, void* out, int32_t dtype, int64_t rows, int64_t cols,
                     const float* scale, int64_t scale_stride, void* stream) {
  if (rows < 0 || cols < 0 || scale_stride < 0) return LCE_ERR_INVALID_ARG;
  if (dtype != LCE_F32 && dtype != LCE_BF16 && dtype != LCE_F16) return LCE_ERR_DTYPE;
  if (rows == 0 || cols == 0) return LCE_OK;
  if (!in || !out || !scale) return LCE_ERR_INVALID_ARG;
  const int64_t vec = dtype == LCE_F32 ? 4 : 8;
  if (!aligned16(in) || !aligned16(out) || (scale_stride != 0 && cols % vec != 0))
    return LCE_ERR_UNSUPPORTED;
  if (rows > INT64_MAX / cols) return LCE_ERR_INVALID_ARG;
  const lce::Elem el = dtype == LCE_BF16 ? lce::Elem::kBF16
                      : dtype == LCE_F16 ? lce::Elem::kF16 : lce::Elem::kF32;
  LCE_HIP(lce::scale(el, in, out, rows * cols, scale_stride == 0 ? 0 : cols,
                     scale, scale_stride, static_cast<hipStream_t>(stream)));
  return LCE_OK;
}

lce_status lce_ce_inplace(float* logits, const int64_t* targets, const float* class_weight,
                          int64_t N, int64_t V, int64_t ignore_index, int32_t reduction,
                          float grad_scale, float* loss, int64_t* n_valid, void* workspace,
                          size_t ws_bytes, void* stream) {
  const lce_status st = ce_check(logits, targets, N, V, reduction, loss);
  if (st != LCE_OK) return st;
  if (!workspace || ws_bytes < ce_scratch_bytes(N) ||
      (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return LCE_ERR_WORKSPACE;
  return ce_enqueue(logits, targets, class_weight, N, V, ignore_index, reduction, grad_scale,
                    loss, n_valid, static_cast<char*>(workspace),
                    static_cast<hipStream_t>(stream));
}

lce_status lce_ce_inplace_noalloc(float* logits, const int64_t* targets,
                                  const float* class_weight, int64_t N, int64_t V,
                                  int64_t ignore_index, int32_t reduction, float grad_scale,
                                  float* loss, int64_t* n_valid, void* stream) {
  const lce_status st = ce_check(logits, targets, N, V, reduction, loss);
  if (st != LCE_OK) return st;
  if (N > LCE_CE_NOALLOC_MAX_ROWS) {
    snprintf(g_last_error, sizeof(g_last_error),
             "lce_ce_inplace_noalloc: N = %lld rows exceeds the static scratch of %lld rows",
             static_cast<long long>(N), static_cast<long long>(LCE_CE_NOALLOC_MAX_ROWS));
    return LCE_ERR_UNSUPPORTED;
  }
  char* ws = nullptr;
  const lce_status sst = noalloc_scratch(&ws);
  if (sst != LCE_OK) return sst;
  return ce_enqueue(logits, targets, class_weight, N, V, ignore_index, reduction, grad_scale,
                    loss, n_valid, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
