// MFMA GEMM tiles for gfx950 (CDNA4).
//
// One workgroup of 256 threads (four 64-wide waves in a 2 x 2 grid) computes a
// 256 x 256 tile of C = A . B^T where both operands keep K contiguous.  Each
// wave owns a 128 x 128 sub-tile held as 4 x 4 accumulator blocks of the
// 32 x 32 MFMA (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2f32 for
// fp32), fp32 accumulation throughout.
//
// K is walked in stages of 128 bytes per row (64 bf16 or 32 fp32).  A stage
// of both operands (2 x 32 KiB) is loaded with 16-byte global loads into
// registers one stage ahead of the MFMAs and written to the other half of a
// double-buffered LDS ring, so one barrier per stage suffices.  Inside LDS the
// eight 16-byte chunks of a row are XOR-swizzled by (row & 7), which makes the
// MFMA fragment reads (32 rows at one chunk position) bank-conflict free.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block id is
// remapped so each XCD walks a contiguous range of tiles, grouped along M, and
// tiles that share an operand slab share that XCD's L2.
//
// The logits GEMM (classes on M, chunk rows on N) carries the fused
// softmax-statistics epilogue: per (row, 256-class tile) max, sum of
// exp(z - max), argmax and the target logit, with exp(z - max) stored as the
// per-chunk tile that becomes the logits gradient in place.  This is the
// chunk loop body of the PyTorch module torch/nn/modules/linear_cross_entropy.py
// (logits mm, bias add, row max subtraction, target gather, sumexp), fused.
#include "lce_kernels.h"

#include <math.h>

namespace lce {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStageBytes = kTile * kStageRowBytes;          // 32 KiB
constexpr int kLdsOperandBytes = 2 * 2 * kStageBytes;        // 128 KiB
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Elt;
template <> struct Elt<uint16_t> { static constexpr int kVec = 8; };
template <> struct Elt<float> { static constexpr int kVec = 4; };

__device__ __forceinline__ float to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float to_f32(float f) { return f; }


__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Block id -> logical tile id such that XCD x (which receives block ids
// x, x + 8, x + 16, ...) walks the contiguous range [x * per, (x + 1) * per).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcds = 8;
  const int per = nblocks / kXcds;
  if (bid >= per * kXcds) return bid;
  return (bid % kXcds) * per + bid / kXcds;
}

// Logical id -> (tile_m, tile_n), walking groups of `group_m` M-tiles across
// all N-tiles, M fastest inside a group.
__device__ __forceinline__ void tile_coords(int logical, int tiles_m, int tiles_n,
                                            int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int grp = logical / per_group;
  const int first = grp * group_m;
  const int gm = min(group_m, tiles_m - first);
  const int idx = logical - grp * per_group;
  tm = first + idx % gm;
  tn = idx / gm;
}

template <typename T>
__device__ __forceinline__ void mfma_step(f32x16_t& acc, i32x4_t a, i32x4_t b);

template <>
__device__ __forceinline__ void mfma_step<uint16_t>(f32x16_t& acc, i32x4_t a, i32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// fp32: a 16-byte fragment holds 4 consecutive k of one row; MFMA q takes
// component q.  Lanes 0-31 hold k = 8s + q and lanes 32-63 k = 8s + 4 + q, so
// the four MFMAs together cover the 8 k of the sub-step exactly once, and A
// and B pair the same k.
template <>
__device__ __forceinline__ void mfma_step<float>(f32x16_t& acc, i32x4_t a, i32x4_t b) {
  const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
  const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
}

// Accumulator layout of a 32 x 32 MFMA block, lane l, register r:
//   column = l & 31, row = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3).
// Wave (wm, wn) owns rows wm*128 + 32 i + ..., columns wn*128 + 32 j + ...

// C tile [m0, m0+256) x [n0, n0+256) += A[m0.., k_begin..k_end) . B[n0.., ...]^T
template <typename T>
__device__ __forceinline__ void mainloop(const T* __restrict__ A, int64_t lda, int m0, int M,
                                         const T* __restrict__ B, int64_t ldb, int n0, int N,
                                         int k_begin, int k_end, char* __restrict__ lds,
                                         f32x16_t (&acc)[4][4]) {
  constexpr int kVec = Elt<T>::kVec;
  constexpr int kBK = kStageRowBytes / static_cast<int>(sizeof(T));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{0};

  const int nk = (k_end - k_begin + kBK - 1) / kBK;
  if (nk <= 0) return;

  // Global -> register mapping: thread t loads chunk (t & 7) of rows
  // (t >> 3) + 32 i, i = 0..7, for each operand.
  const int ch = tid & 7;
  const int r0 = tid >> 3;
  const T* pa = A + static_cast<int64_t>(m0 + r0) * lda + ch * kVec;
  const T* pb = B + static_cast<int64_t>(n0 + r0) * ldb + ch * kVec;
  const int64_t sa = 32 * lda, sb = 32 * ldb;
  const int st_off = r0 * kStageRowBytes + ((ch ^ (r0 & 7)) << 4);

  i32x4_t ga[8], gb[8];
  auto gload = [&](int k0) {
    const bool kin = (k0 + ch * kVec) < k_end;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ga[i] = i32x4_t{0, 0, 0, 0};
      gb[i] = i32x4_t{0, 0, 0, 0};
      if (kin && m0 + r0 + 32 * i < M)
        ga[i] = *reinterpret_cast<const i32x4_t*>(pa + i * sa + k0);
      if (kin && n0 + r0 + 32 * i < N)
        gb[i] = *reinterpret_cast<const i32x4_t*>(pb + i * sb + k0);
    }
  };
  auto sstore = [&](int stage) {
    char* la = lds + stage * (2 * kStageBytes);
    char* lb = la + kStageBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<i32x4_t*>(la + st_off + i * 32 * kStageRowBytes) = ga[i];
      *reinterpret_cast<i32x4_t*>(lb + st_off + i * 32 * kStageRowBytes) = gb[i];
    }
  };

  // Fragment reads: lane l reads row (l & 31) of each 32-row block at chunk
  // (2 kk + (l >> 5)) of the stage, swizzled by (row & 7) = (l & 7).
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  const int fsw = lane & 7;
  const int a_row = (wm * 128 + frow) * kStageRowBytes;
  const int b_row = (wn * 128 + frow) * kStageRowBytes;

  gload(k_begin);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(k_begin + (kt + 1) * kBK);
    const char* la = lds + cur * (2 * kStageBytes);
    const char* lb = la + kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = ((2 * kk + fhalf) ^ fsw) << 4;
      i32x4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const i32x4_t*>(la + a_row + i * 32 * kStageRowBytes + c);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const i32x4_t*>(lb + b_row + j * 32 * kStageRowBytes + c);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_step<T>(acc[i][j], af[i], bf[j]);
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- plain GEMM
// The output is stored transposed, C[n * ldc + m]: lane l holds 4
// consecutive m (registers 4q..4q+3) of column n, so every store (and every
// load of the accumulate modes) is one 16-byte (fp32) or 8-byte (bf16)
// vector.  M must be a multiple of 4.
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef f32x4_t type; };
template <> struct Vec4<uint16_t> { typedef bf16x4_t type; };

template <typename T>
__device__ __forceinline__ f32x4_t load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else {
    const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
    return f32x4_t{static_cast<float>(v[0]), static_cast<float>(v[1]),
                   static_cast<float>(v[2]), static_cast<float>(v[3])};
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4_t v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4_t*>(p) = v;
  } else {
    bf16x4_t o;
    o[0] = static_cast<__bf16>(v[0]);
    o[1] = static_cast<__bf16>(v[1]);
    o[2] = static_cast<__bf16>(v[2]);
    o[3] = static_cast<__bf16>(v[3]);
    *reinterpret_cast<bf16x4_t*>(p) = o;
  }
}

template <typename T, int kMode>
__global__ __launch_bounds__(kThreads) void k_gemm_nt(GemmNT g) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsOperandBytes];
  const int tiles_m = cdiv(g.M, kTile), tiles_n = cdiv(g.N, kTile);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = tiles_m * tiles_n;
  const int split = logical / per_split;
  int tm, tn;
  tile_coords(logical - split * per_split, tiles_m, tiles_n, g.group_m, tm, tn);
  const int kb = split * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  f32x16_t acc[4][4];
  mainloop<T>(static_cast<const T*>(g.A), g.lda, tm * kTile, g.M,
              static_cast<const T*>(g.B), g.ldb, tn * kTile, g.N, kb, ke, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int mb = tm * kTile + wm * 128 + 4 * (lane >> 5);
  const int nb = tn * kTile + wn * 128 + (lane & 31);
  const int64_t ldc = g.ldc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nb + 32 * j;
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = mb + 32 * i + 8 * q;
        if (m >= g.M) continue;
        const int64_t off = static_cast<int64_t>(n) * ldc + m;
        f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                     acc[i][j][4 * q + 3]};
        if constexpr (kMode == static_cast<int>(EpiMode::kStoreF32)) {
          store4(static_cast<float*>(g.C) + split * g.split_stride + off, v);
        } else if constexpr (kMode == static_cast<int>(EpiMode::kAccumF32)) {
          float* c = static_cast<float*>(g.C) + off;
          store4(c, load4(c) + v);
        } else if constexpr (kMode == static_cast<int>(EpiMode::kFinalOut)) {
          store4(static_cast<T*>(g.C) + off, load4(static_cast<const float*>(g.Cin) + off) + v);
        } else if constexpr (kMode == static_cast<int>(EpiMode::kStoreOut)) {
          store4(static_cast<T*>(g.C) + off, v);
        } else {
          T* c = static_cast<T*>(g.C) + off;
          store4(c, load4(c) + v);
        }
      }
  }
}

// ------------------------------------------------- logits + softmax stats
template <typename T, bool kStoreT, bool kArgmax>
__global__ __launch_bounds__(kThreads) void k_logits_lse(LogitsLse a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsOperandBytes];
  __shared__ float red_m[2][kTile];
  __shared__ int red_i[2][kTile];
  __shared__ float red_s[2][kTile];

  const int tiles_m = cdiv(a.V, kTile), tiles_n = cdiv(a.rows, kTile);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_coords(logical, tiles_m, tiles_n, 4, tm, tn);

  f32x16_t acc[4][4];
  // M = classes (rows of W), N = chunk rows (rows of X), K = D.
  mainloop<T>(static_cast<const T*>(a.W), a.ldw, tm * kTile, a.V,
              static_cast<const T*>(a.X), a.ldx, tn * kTile, a.rows, 0, a.D, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fhalf = lane >> 5;
  const int vbase = tm * kTile + wm * 128;               // class of (i=0, r=0, half 0)
  const int vlane = vbase + 4 * fhalf;                   // + 32 i + 8 (r >> 2) + (r & 3)
  const int ncol = wn * 128 + frow;                      // + 32 j, within the tile
  const int nbase = tn * kTile + ncol;
  const T* bias = static_cast<const T*>(a.bias);

  // 1. bias, and -inf for classes beyond V.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vlane + 32 * i + 8 * (r >> 2) + (r & 3);
      const bool in = v < a.V;
      const float bb = (in && bias) ? to_f32(bias[v]) : 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j][r] = in ? acc[i][j][r] + bb : -INFINITY;
    }

  // 2. target logit: the lane holding class tc[n] of column n writes zt[n].
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nbase + 32 * j;
    if (n < a.rows) {
      const int t = a.tc[n];
      const int off = t - vbase;
      if (t >= 0 && off >= 0 && off < 128 && ((off >> 2) & 1) == fhalf) {
        const int want = ((off >> 5) << 4) | (((off >> 3) & 3) << 2) | (off & 3);
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) val = (i * 16 + r == want) ? acc[i][j][r] : val;
        a.zt[n] = val;
      }
    }
  }

  // 3. column max (and lowest class attaining it) over the tile's 256 classes.
  float cmax[4];
  int cidx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = -INFINITY;
    int mi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = acc[i][j][r];
        if (z > mx) {
          mx = z;
          if constexpr (kArgmax) mi = vlane + 32 * i + 8 * (r >> 2) + (r & 3);
        }
      }
    const float om = __shfl_xor(mx, 32);
    const int oi = __shfl_xor(mi, 32);
    if (om > mx || (om == mx && oi < mi)) {
      mx = om;
      mi = oi;
    }
    cmax[j] = mx;
    cidx[j] = mi;
    if (fhalf == 0) {
      red_m[wm][ncol + 32 * j] = mx;
      red_i[wm][ncol + 32 * j] = mi;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float om = red_m[wm ^ 1][ncol + 32 * j];
    const int oi = red_i[wm ^ 1][ncol + 32 * j];
    if (om > cmax[j] || (om == cmax[j] && oi < cidx[j])) {
      cmax[j] = om;
      cidx[j] = oi;
    }
  }

  // 4. e = exp(z - tile max) in place, column sums.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mx = cmax[j];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // (z - max) first: the maximum maps to exactly 1.
        const float e = __builtin_amdgcn_exp2f((acc[i][j][r] - mx) * kLog2e);
        acc[i][j][r] = e;
        s += e;
      }
    s += __shfl_xor(s, 32);
    if (fhalf == 0) red_s[wm][ncol + 32 * j] = s;
  }
  __syncthreads();

  // 5. per-(row, class tile) statistics.
  if (wm == 0 && fhalf == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nbase + 32 * j;
      if (n < a.rows) {
        const int64_t o = static_cast<int64_t>(tm) * a.ldp + n;
        a.m_part[o] = cmax[j];
        a.s_part[o] = red_s[0][ncol + 32 * j] + red_s[1][ncol + 32 * j];
        if constexpr (kArgmax) a.i_part[o] = cidx[j];
      }
    }
  }

  // 6. the exp tile T[n][v], 4 consecutive classes per store.
  if constexpr (kStoreT) {
    T* Tm = static_cast<T*>(a.T);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nbase + 32 * j;
      if (n >= a.rows) continue;
      T* row = Tm + static_cast<int64_t>(n) * a.ldt;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v0 = vlane + 32 * i + 8 * q;
          if constexpr (sizeof(T) == 2) {
            bf16x4_t pk;
            pk[0] = static_cast<__bf16>(acc[i][j][4 * q + 0]);
            pk[1] = static_cast<__bf16>(acc[i][j][4 * q + 1]);
            pk[2] = static_cast<__bf16>(acc[i][j][4 * q + 2]);
            pk[3] = static_cast<__bf16>(acc[i][j][4 * q + 3]);
            *reinterpret_cast<bf16x4_t*>(row + v0) = pk;
          } else {
            f32x4_t pk = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
                          acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(row + v0) = pk;
          }
        }
    }
  }
}

template <typename T>
hipError_t launch_gemm(const GemmNT& g, hipStream_t s) {
  const int tiles = ((g.M + kTile - 1) / kTile) * ((g.N + kTile - 1) / kTile) * g.splits;
  if (tiles <= 0) return hipSuccess;
  const dim3 grid(tiles), block(kThreads);
  switch (g.mode) {
    case EpiMode::kStoreF32: k_gemm_nt<T, 0><<<grid, block, 0, s>>>(g); break;
    case EpiMode::kAccumF32: k_gemm_nt<T, 1><<<grid, block, 0, s>>>(g); break;
    case EpiMode::kFinalOut: k_gemm_nt<T, 2><<<grid, block, 0, s>>>(g); break;
    case EpiMode::kStoreOut: k_gemm_nt<T, 3><<<grid, block, 0, s>>>(g); break;
    case EpiMode::kAccumOut: k_gemm_nt<T, 4><<<grid, block, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_logits(const LogitsLse& a, hipStream_t s) {
  const int tiles = ((a.V + kTile - 1) / kTile) * ((a.rows + kTile - 1) / kTile);
  if (tiles <= 0) return hipSuccess;
  const dim3 grid(tiles), block(kThreads);
  const bool st = a.T != nullptr, am = a.i_part != nullptr;
  if (st && am) k_logits_lse<T, true, true><<<grid, block, 0, s>>>(a);
  else if (st) k_logits_lse<T, true, false><<<grid, block, 0, s>>>(a);
  else if (am) k_logits_lse<T, false, true><<<grid, block, 0, s>>>(a);
  else k_logits_lse<T, false, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_nt(bool bf16, const GemmNT& g, hipStream_t s) {
  return bf16 ? launch_gemm<uint16_t>(g, s) : launch_gemm<float>(g, s);
}

hipError_t logits_lse(bool bf16, const LogitsLse& a, hipStream_t s) {
  return bf16 ? launch_logits<uint16_t>(a, s) : launch_logits<float>(a, s);
}

}  // namespace lce
