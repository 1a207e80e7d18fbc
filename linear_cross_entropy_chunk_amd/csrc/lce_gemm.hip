// MFMA GEMM tiles for gfx950 (CDNA4).
//
// One workgroup of 256 threads (four 64-wide waves, one per SIMD, in a 2 x 2
// grid) computes a 256 x 256 tile of P = A . B^T where both operands keep K
// contiguous.  Each wave owns a 128 x 128 sub-tile held as 8 x 8 accumulator
// blocks of the 16 x 16 MFMA (v_mfma_f32_16x16x32_bf16 for bf16,
// v_mfma_f32_16x16x4f32 for fp32) in the 256 accumulation registers, fp32
// accumulation throughout.  The 16 x 16 shape moves a quarter of the
// accumulator bytes per flop of the 32 x 32 one; the chip runs these tiles
// at its power limit, where that is worth several percent of clock.
//
// K is walked in stages of 128 bytes per row (64 bf16 or 32 fp32).  Operand
// tiles go from global memory straight into LDS (buffer_load_dwordx4 ... lds),
// each instruction moving eight whole 128-byte rows, i.e. whole L2 lines.
// The 160 KiB of LDS form five 32 KiB slots, one operand of one stage each:
// stage s keeps A in slot 2s mod 5 and B in slot 2s + 1 mod 5, so while stage
// s is consumed, B of stage s + 1 and A of stage s + 2 are in flight.  Copies
// are spread over the MFMA stream to keep the per-CU address unit below
// saturation, and there is one barrier per stage.
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
#include "lce_device.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace lce {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Wave layout of a 256 x 256 tile: kWavesM x kWavesN waves (one per SIMD),
// each owning a 128 x 128 sub-tile of kI x kJ blocks of 16 x 16.
constexpr int kWavesM = 2;
constexpr int kWavesN = 2;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveM = kTile / kWavesM;       // rows per wave
constexpr int kWaveN = kTile / kWavesN;       // columns per wave
constexpr int kBlk = 16;                      // MFMA block edge
constexpr int kI = kWaveM / kBlk;             // 8 row blocks per wave
constexpr int kJ = kWaveN / kBlk;             // 8 column blocks per wave
constexpr int kRowBytes = 128;                // bytes per row per K stage
constexpr int kSlotBytes = kTile * kRowBytes; // one operand of one stage: 32 KiB
constexpr int kSlots = 5;
constexpr int kLdsOperandBytes = kSlots * kSlotBytes;        // 160 KiB ring
constexpr int kCopies = kTile / 8 / kWaves;   // 8-row copies per operand per wave per stage
constexpr uint32_t kRepairGrid = 256;         // workgroups of the gated repair pass (one per CU)
constexpr float kLog2e = 1.4426950408889634f;

// Accumulator layout of a 16 x 16 MFMA block, lane l, register r:
//   column = l & 15, row = 4 (l >> 4) + r.
// Wave (wm, wn) owns rows wm * 128 + 16 i + ..., columns wn * 128 + 16 j + ...
typedef f32x4_t Acc[kI][kJ];

// One element of type T at byte offset `off` of a buffer, as fp32 (0 past
// the descriptor's range).
template <typename T>
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  } else if constexpr (std::is_same_v<T, _Float16>) {
    return static_cast<float>(
        __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0)));
  } else {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0))
                           << 16);
  }
}

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

// One pair of 16-byte fragments.  Lane l holds row l & 15 of its 16-row
// block at the logical chunk 4 h + (l >> 4) of sub-step h.
//   bf16 / fp16: the chunk is k = 8 (l >> 4) .. + 7 of the sub-step, exactly
//         the operand of v_mfma_f32_16x16x32_bf16 / _f16.
//   fp32: the chunk holds 4 consecutive k; MFMA p takes component p, so lane
//         group q supplies k = 4 q + p and the four MFMAs cover the 16 k of
//         the sub-step once, with A and B paired on the same k.
template <typename T>
__device__ __forceinline__ void mfma_step(f32x4_t& acc, i32x4_t a, i32x4_t b);

template <>
__device__ __forceinline__ void mfma_step<uint16_t>(f32x4_t& acc, i32x4_t a, i32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<_Float16>(f32x4_t& acc, i32x4_t a, i32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(f32x4_t& acc, i32x4_t a, i32x4_t b) {
  const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
  const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], acc, 0, 0, 0);
}

using dev::make_rsrc;
using dev::kOutOfRange;

// ------------------------------------------------------------- main loop
// LDS layout of a slot: row r of the 256-row operand tile at byte 128 r; its
// 16-byte chunk with logical index c sits at physical chunk c ^ ((r >> 1) & 7).
// A ds_read_b128 serves 16 lanes per cycle, and the fragment reads put 16
// consecutive rows at one logical chunk in such a group: with 128-byte rows
// the bank group of (r, p) is 8 (r & 1) + p, and the swizzle makes those 16
// distinct.  The copy applies the inverse on the global side: lane i of a
// copy instruction fetches logical chunk (i & 7) ^ swz(row) of row i / 8.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

using dev::copy16_to_lds;
using dev::lds_addr;
using dev::waitcnt_vm;
constexpr int kWaitVm0 = waitcnt_vm(0);

// A k-major operand (stored [K][ld], its M or N index contiguous, bf16)
// keeps a stage in a slot as 64 k-rows of 512 bytes (256 columns); the
// 16-byte chunk c of k-row r sits at physical chunk c ^ trswz(r).  Fragments
// come from ds_read_b64_tr_b16: within each group of 16 lanes, source lane s
// supplies 4 consecutive columns of one k-row and output lane l receives
// column l & 3 of source lanes 4e + l / 4 (e = 0..3), i.e. four consecutive k
// of one column -- two such reads give the 16x16x32 operand of a lane
// (column l & 15, k = 8 (l >> 4) .. + 7).  A 16-lane group reads 32 bytes from
// each of four consecutive k-rows and two groups go per cycle; trswz spreads
// those eight 32-byte pieces over all 64 banks.
__device__ __forceinline__ int trswz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ i32x4_t read_tr_pair(const char* lds_p) {
  typedef __attribute__((address_space(3))) char lds_char_t;
  lds_char_t* base = reinterpret_cast<lds_char_t*>(static_cast<uintptr_t>(dev::lds_addr(lds_p)));
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4_t*>(base));
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4_t*>(base + 4 * 512));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(i32x4_t, v);
}

// C tile [m0, m0+256) x [n0, n0+256) = A[m0.., k_begin..k_end) . B[n0.., ...]^T
// (added to the accumulators' values on entry with kAccInit, else from zero)
//
// Rows past M (N) read as zero (each copy's descriptor covers only the
// tile's existing rows); so do k-rows of a k-major operand past its valid
// rows.  With kKTail, 16-byte chunks at or past k_end read as zero too
// (their offsets are sent out of range; K-contiguous operands only).
// With kBPan, B lies in the T panel layout (ldb = kTile, panel stride b_ps):
// K-contiguous, a stage's 64 k sit in panel k0 / kTile and the copy's
// descriptor starts at that panel's tile rows; k-major, the tile's kTile
// columns are one panel and the descriptor starts at its k-row k0.
//
// Per stage s (two sub-steps of 4 chunks, 64 MFMAs per wave each), every wave:
//   sub-step 0 and the first quarter of sub-step 1: MFMAs from registers;
//     the 16 LDS reads of sub-step 1 (during sub-step 0, one per 4 MFMAs);
//     8 copies of A of stage s + 2 into slot 2s + 4 mod 5 (the slot B of
//     stage s - 1 left), one per 8 MFMAs and never in a read's slot;
//   wait for its copies of stage s + 1 (all but the 8 just issued) and for
//   its LDS reads; barrier: stage s + 1 is whole and stage s is fully read;
//   the rest of sub-step 1: MFMAs; the 16 LDS reads of sub-step 0 of stage
//     s + 1 (one per 3 MFMAs); 8 copies of B of stage s + 2 into slot 2s mod
//     5 (one per 6 MFMAs, again in slots of their own).
// A stage's B thus has most of a stage to land and its A about seven
// quarters.  An MFMA slot carries at most one read or one copy: a slot with
// both stretches the gap between two MFMAs past the 16 cycles one takes.
template <typename T, bool kKTail, bool kATr, bool kBTr, bool kBPan = false,
          bool kAccInit = false>
__device__ __forceinline__ void mainloop(const T* __restrict__ A, int64_t lda, int m0, int M,
                                         int a_krows,
                                         const T* __restrict__ B, int64_t ldb, int n0, int N,
                                         int b_krows, int64_t b_ps,
                                         int k_begin, int k_end, char* __restrict__ lds,
                                         Acc& acc) {
  static_assert(kI == 8 && kJ == 8 && kWaves == 4 && kCopies == 8, "four waves of 128 x 128");
  static_assert(!(kATr || kBTr) || sizeof(T) == 2, "k-major operands are 2-byte types only");
  static_assert(!(kKTail && (kATr || kBTr)), "k tails apply to K-contiguous operands");
  static_assert(!(kKTail && kBPan), "panels hold whole stages");
  constexpr int kEs = static_cast<int>(sizeof(T));
  constexpr int kBK = kRowBytes / kEs;            // K elements per stage
  constexpr int kVec = 16 / kEs;                  // elements per 16-byte chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: copy bases in SGPRs
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  if constexpr (!kAccInit) {   // kAccInit: the caller has loaded the accumulators
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < kJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int nk = (k_end - k_begin + kBK - 1) / kBK;
  if (nk <= 0) return;

  // K-contiguous operand: one descriptor over the tile's rows.  Copy j of a
  // wave covers rows 8 (kCopies wave + j) .. + 8; lane i takes row + i / 8,
  // physical chunk i & 7.  The stage's K offset travels in the instruction's
  // scalar offset.
  // k-major operand: copy j covers k-rows 2 (kCopies wave + j) .. + 2 of the
  // stage; lane i takes k-row + i / 32, physical chunk i & 31.  The
  // descriptor is rebased on the stage's first k-row.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda,
                                              static_cast<int64_t>(min(M - m0, kTile)) * lda * kEs);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + static_cast<int64_t>(n0) * ldb,
                                              static_cast<int64_t>(min(N - n0, kTile)) * ldb * kEs);
  auto lane_off = [&](bool tr, int64_t ld, int j) {
    if (tr) {
      const int r = 2 * (kCopies * wave + j) + (lane >> 5);
      return (r * static_cast<int>(ld) + (((lane & 31) ^ trswz(r)) << 3)) * kEs;
    }
    const int row = 8 * (kCopies * wave + j) + (lane >> 3);
    return (row * static_cast<int>(ld) + (((lane & 7) ^ swz(row)) * kVec)) * kEs;
  };
  int va[kCopies], vb[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    va[j] = lane_off(kATr, lda, j);
    vb[j] = lane_off(kBTr, ldb, j);
  }
  // a descriptor whose fields are visibly uniform, so that it lives in SGPRs
  auto uniform_rsrc = [](const T* p, int64_t bytes) {
    const uint64_t addr = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
    const int range = __builtin_amdgcn_readfirstlane(
        bytes > 0x7ffff000LL * 2 ? -1 : static_cast<int>(static_cast<uint32_t>(bytes)));
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, range, 0x00020000);
  };
  // Where the copies of one operand of one stage read: a descriptor and a
  // scalar offset, fixed for the stage.  They are formed in an MFMA slot of
  // their own ahead of the stage's first copy, so that no copy slot carries
  // the address arithmetic (a 64-bit product and clamps for the k-major and
  // panel operands).
  struct Src {
    __amdgpu_buffer_rsrc_t rs;
    int soff;
    int k0;
  };
  auto src_of = [&](int st, bool opb) -> Src {
    const int k0 = k_begin + min(st, nk - 1) * kBK;   // stages past the end repeat the last
    const bool tr = opb ? kBTr : kATr;
    if (kBPan && opb && !kBTr) {
      // the tile's rows of panel k0 / kTile; rows past N read as zero
      const T* base = B + (k0 / kTile) * b_ps + static_cast<int64_t>(n0) * kTile;
      const int64_t bytes = static_cast<int64_t>(min(N - n0, kTile)) * kTile * kEs;
      return Src{uniform_rsrc(base, bytes), __builtin_amdgcn_readfirstlane((k0 % kTile) * kEs),
                 k0};
    } else if (kBPan && opb) {
      // k-major panel of the tile's columns: k-rows from k0 to b_krows
      const T* base = B + (n0 / kTile) * b_ps + static_cast<int64_t>(k0) * kTile;
      const int64_t bytes = static_cast<int64_t>(max(b_krows - k0, 0)) * kTile * kEs;
      return Src{uniform_rsrc(base, bytes), 0, k0};
    } else if (tr) {
      const T* base = opb ? B + n0 : A + m0;
      const int64_t ld = opb ? ldb : lda;
      const int krows = opb ? b_krows : a_krows;
      const int64_t left = (static_cast<int64_t>(max(krows - k0, 0)) * ld - (opb ? n0 : m0)) * kEs;
      return Src{uniform_rsrc(base + static_cast<int64_t>(k0) * ld, left > 0 ? left : 0), 0, k0};
    }
    return Src{opb ? rb : ra, __builtin_amdgcn_readfirstlane(k0 * kEs), k0};
  };
  auto copy = [&](const Src& src, int slot, bool opb, int j) {
    const uint32_t dst = lds_addr(lds + slot * kSlotBytes + (kCopies * wave + j) * 1024);
    int o = opb ? vb[j] : va[j];
    if constexpr (kKTail) {                   // K-contiguous operands only
      const int row = 8 * (kCopies * wave + j) + (lane >> 3);
      o = (src.k0 + ((lane & 7) ^ swz(row)) * kVec) < k_end ? o : kOutOfRange;
    }
    copy16_to_lds(src.rs, o, dst, src.soff);
  };

  // Fragment reads of a K-contiguous operand: lane l reads row (l & 15) of
  // each 16-row block at logical chunk 4 h + (l >> 4) of sub-step h.  Rows
  // 16 x + (l & 15) share the swizzle of (l & 15).
  // Fragment reads of a k-major operand: see trswz; lane l (group g = l / 16,
  // s = l & 15) reads k-rows 32 h + 8 g + 4 rd + s / 4 (rd = 0, 1) at columns
  // 16 x + 4 (s & 3) .. + 3 of its wave's 128.
  // Read r (0..15) of a sub-step: A block r / 2 if r is even, else B block r / 2.
  const int frow = lane & 15, fq = lane >> 4, fsw = swz(frow);
  int coff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) coff[h] = ((4 * h + fq) ^ fsw) << 4;
  auto tr_off = [&](int wpos, int x) {   // byte offset of block x, sub-step 0, rd 0
    const int s4 = lane & 15;
    const int krow = 8 * fq + (s4 >> 2);
    const int lc = 16 * wpos + 2 * x + ((s4 & 3) >> 1);
    return krow * 512 + ((lc ^ trswz(krow)) << 4) + (s4 & 1) * 8;
  };
  int ta[kATr ? kI : 1], tb[kBTr ? kJ : 1];
#pragma unroll
  for (int x = 0; x < (kATr ? kI : 1); ++x) ta[x] = kATr ? tr_off(wm, x) : 0;
#pragma unroll
  for (int x = 0; x < (kBTr ? kJ : 1); ++x) tb[x] = kBTr ? tr_off(wn, x) : 0;
  const int a_row = (wm * kWaveM + frow) * kRowBytes;
  const int b_row = (wn * kWaveN + frow) * kRowBytes;
  i32x4_t af[2][kI], bf[2][kJ];
  auto read = [&](int sa, int sb, int h, int set, int r) {
    const int x = r >> 1;
    if (r & 1) {
      if constexpr (kBTr)
        bf[set][x] = read_tr_pair(lds + sb * kSlotBytes + tb[x] + h * 32 * 512);
      else
        bf[set][x] = *reinterpret_cast<const i32x4_t*>(lds + sb * kSlotBytes + b_row + coff[h] +
                                                       x * kBlk * kRowBytes);
    } else {
      if constexpr (kATr)
        af[set][x] = read_tr_pair(lds + sa * kSlotBytes + ta[x] + h * 32 * 512);
      else
        af[set][x] = *reinterpret_cast<const i32x4_t*>(lds + sa * kSlotBytes + a_row + coff[h] +
                                                       x * kBlk * kRowBytes);
    }
  };
  auto mfma = [&](int set, int u) {     // u = 8 i + j
    mfma_step<T>(acc[u >> 3][u & 7], af[set][u >> 3], bf[set][u & 7]);
  };

  // Prologue: stages 0 and 1 whole (slots 0-3), stage 0 landed.
  {
    const Src a0 = src_of(0, false), b0 = src_of(0, true);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) { copy(a0, 0, false, j); copy(b0, 1, true, j); }
    const Src a1 = src_of(1, false), b1 = src_of(1, true);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) { copy(a1, 2, false, j); copy(b1, 3, true, j); }
  }
  // the sources of stage s + 2's copies, formed a few slots ahead of them
  Src src_a = src_of(2, false), src_b = src_of(2, true);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopies));
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) read(0, 1, 0, 0, r);

  // One stage; r5 = s mod 5 is a compile-time constant so every slot index is.
  // The order of MFMAs, LDS reads and copies is pinned with scheduling
  // barriers: every slot of the MFMA stream carries at most one read or one
  // copy.
  auto stage = [&](auto rc, int kt) {
    constexpr int r5 = decltype(rc)::value;
    const int s = kt + r5;
    if (s >= nk) return;                                   // uniform
    constexpr int sa = (2 * r5) % kSlots, sb = (2 * r5 + 1) % kSlots;
    constexpr int na = (2 * r5 + 2) % kSlots, nb = (2 * r5 + 3) % kSlots;
    constexpr int ca = (2 * r5 + 4) % kSlots, cb = (2 * r5 + 5) % kSlots;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 80; ++t) {          // sub-step 0, first quarter of sub-step 1
      mfma(t >> 6, t & 63);
      if (t < 64 && t % 8 == 2) copy(src_a, ca, false, t / 8);
      if (t < 64 && t % 4 == 0) read(sa, sb, 1, 1, t / 4);
      if (t == 5) src_b = src_of(s + 2, true);             // an empty slot
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopies) & ~0x0f00);   // vmcnt(8) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 16; u < 64; ++u) {         // rest of sub-step 1
      mfma(1, u);
      if ((u - 16) % 6 == 1) copy(src_b, cb, true, (u - 17) / 6);
      if ((u - 16) % 3 == 0) read(na, nb, 0, 0, (u - 16) / 3);
      if (u == 20) src_a = src_of(s + 3, false);           // an empty slot: next stage's A
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk; kt += kSlots) {
    stage(std::integral_constant<int, 0>{}, kt);
    stage(std::integral_constant<int, 1>{}, kt);
    stage(std::integral_constant<int, 2>{}, kt);
    stage(std::integral_constant<int, 3>{}, kt);
    stage(std::integral_constant<int, 4>{}, kt);
  }
  // Drain the copies still in flight before the LDS is reused.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
}

// ---------------------------------------------------------------- plain GEMM
// The output is stored transposed, C[n * ldc + m]: lane l holds 4
// consecutive m (registers 0..3) of column n, so every store (and every load
// of the accumulate modes) is one 16-byte (fp32) or 8-byte (bf16, fp16) vector, and
// the four lane groups of a column cover 16 consecutive m.  M must be a
// multiple of 4.
template <typename T>
__device__ __forceinline__ f32x4_t load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else if constexpr (std::is_same_v<T, _Float16>) {
    const f16x4_t v = *reinterpret_cast<const f16x4_t*>(p);
    return f32x4_t{static_cast<float>(v[0]), static_cast<float>(v[1]),
                   static_cast<float>(v[2]), static_cast<float>(v[3])};
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
  } else if constexpr (std::is_same_v<T, _Float16>) {
    f16x4_t o;
    o[0] = static_cast<_Float16>(v[0]);
    o[1] = static_cast<_Float16>(v[1]);
    o[2] = static_cast<_Float16>(v[2]);
    o[3] = static_cast<_Float16>(v[3]);
    *reinterpret_cast<f16x4_t*>(p) = o;
  } else {
    bf16x4_t o;
    o[0] = static_cast<__bf16>(v[0]);
    o[1] = static_cast<__bf16>(v[1]);
    o[2] = static_cast<__bf16>(v[2]);
    o[3] = static_cast<__bf16>(v[3]);
    *reinterpret_cast<bf16x4_t*>(p) = o;
  }
}

// 16-bit outputs: two accumulator blocks i0 = 2p and i1 = 2p + 1 of one
// column (lane group q holds M values 4q .. 4q + 3 of each 16-value block),
// rounded to the element type and traded between lane groups q and q ^ 1
// with v_permlane16_swap (vdst's rows 1 and 3 swap with src's rows 0 and 2;
// lane layout checked on the chip).  Afterwards lane group q holds the 8
// consecutive M values pair_off(p, q) .. + 7 of the pair's 32, so a column's
// 32 values leave in four 16-byte stores instead of eight 8-byte ones.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ uint2 pack4(f32x4_t v) {
  static_assert(sizeof(T) == 2, "16-bit element types");
  if constexpr (std::is_same_v<T, _Float16>) {
    f16x4_t o;
    o[0] = static_cast<_Float16>(v[0]);
    o[1] = static_cast<_Float16>(v[1]);
    o[2] = static_cast<_Float16>(v[2]);
    o[3] = static_cast<_Float16>(v[3]);
    return __builtin_bit_cast(uint2, o);
  } else {
    bf16x4_t o;
    o[0] = static_cast<__bf16>(v[0]);
    o[1] = static_cast<__bf16>(v[1]);
    o[2] = static_cast<__bf16>(v[2]);
    o[3] = static_cast<__bf16>(v[3]);
    return __builtin_bit_cast(uint2, o);
  }
}

template <typename T>
__device__ __forceinline__ u32x4_t pair_rows8(f32x4_t v0, f32x4_t v1) {
  const uint2 a = pack4<T>(v0), b = pack4<T>(v1);
  const auto x = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  return u32x4_t{x[0], y[0], x[1], y[1]};
}

__device__ __forceinline__ int pair_off(int p, int q) { return 16 * (2 * p + (q & 1)) + 8 * (q >> 1); }

template <typename T, int kMode, bool kATr, bool kBTr, bool kBPan>
__device__ __forceinline__ void gemm_nt_tile(const GemmNT& g) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsOperandBytes];
  const int tiles_m = cdiv(g.M, kTile), tiles_n = cdiv(g.N, kTile);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = tiles_m * tiles_n;
  const int split = logical / per_split;
  int tm, tn;
  tile_coords(logical - split * per_split, tiles_m, tiles_n, g.group_m, tm, tn);
  const int kb = split * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int mb = tm * kTile + wm * kWaveM + 4 * (lane >> 4);
  const int nb = tn * kTile + wn * kWaveN + (lane & 15);
  const int64_t ldc = g.ldc;
  const float osc = g.out_scale ? g.out_scale[0] : 1.0f;   // product scale, element-type stores

  // The fp32 read-modify-write modes start the accumulators from the fp32
  // values in memory instead of reading them in the epilogue: these loads
  // overlap the wait for the tile's first operand stage, where an epilogue
  // read would come when every tile of a wave finishes at once.  The loads
  // are unconditional, through a descriptor over the tile's rows of the
  // stored matrix (rows past N read as 0; columns past M read neighbouring
  // values that are never stored), so they go straight to the accumulation
  // registers.
  constexpr bool kInit = kMode == static_cast<int>(EpiMode::kAccumF32) ||
                         kMode == static_cast<int>(EpiMode::kFinalOut);
  Acc acc;
  if constexpr (kInit) {
    const float* src = static_cast<const float*>(
        kMode == static_cast<int>(EpiMode::kFinalOut) ? g.Cin : g.C);
    const int n0 = tn * kTile, m0 = tm * kTile;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        src + static_cast<int64_t>(n0) * ldc + m0,
        (static_cast<int64_t>(min(g.N - n0, kTile)) * ldc - m0) * 4);
    const int nl = wn * kWaveN + (lane & 15), ml = wm * kWaveM + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int i = 0; i < kI; ++i)
        acc[i][j] = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, ((nl + kBlk * j) * static_cast<int>(ldc) + ml + kBlk * i) * 4, 0, 0));
  }
  mainloop<T, false, kATr, kBTr, kBPan, kInit>(static_cast<const T*>(g.A), g.lda, tm * kTile,
                                               g.M, g.a_krows, static_cast<const T*>(g.B), g.ldb,
                                               tn * kTile, g.N, g.b_krows, g.b_pstride, kb, ke,
                                               lds, acc);

  constexpr bool kWide = sizeof(T) == 2 && (kMode == static_cast<int>(EpiMode::kStoreOut) ||
                                            kMode == static_cast<int>(EpiMode::kFinalOut));
  // Column factors of the element-type store modes, all eight loaded at once.
  constexpr bool kColScale = kMode == static_cast<int>(EpiMode::kStoreOut) ||
                             kMode == static_cast<int>(EpiMode::kAccumOut);
  float csc[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) csc[j] = osc;
  if constexpr (kColScale) {
    if (g.n_scale) {
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int n = nb + kBlk * j;
        if (n < g.N) csc[j] = osc * g.n_scale[n];
      }
    }
  }
  if constexpr (kWide) {
    // M is a multiple of 8 for 16-bit types, so a lane's 8 values are all
    // inside M or all outside.  The trade pairs lanes of the same column,
    // which share the n test.
    const int mw = tm * kTile + wm * kWaveM;
    const int q = lane >> 4;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      // Column blocks not yet stored stay in the accumulator registers, so
      // only one block's values are copied to VGPRs at a time.
#pragma unroll
      for (int jj = j + 1; jj < kJ; ++jj)
#pragma unroll
        for (int i = 0; i < kI; ++i) asm volatile("" : "+a"(acc[i][jj]));
      const int n = nb + kBlk * j;
      if (n >= g.N) continue;
#pragma unroll
      for (int p = 0; p < kI / 2; ++p) {
        const u32x4_t w = pair_rows8<T>(acc[2 * p][j] * csc[j], acc[2 * p + 1][j] * csc[j]);
        const int m = mw + pair_off(p, q);
        if (m < g.M)
          *reinterpret_cast<u32x4_t*>(static_cast<T*>(g.C) + static_cast<int64_t>(n) * ldc + m) = w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
#pragma unroll
    for (int jj = j + 1; jj < kJ; ++jj)   // blocks not yet stored stay in AGPRs
#pragma unroll
      for (int i = 0; i < kI; ++i) asm volatile("" : "+a"(acc[i][jj]));
    const int n = nb + kBlk * j;
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < kI; ++i) {
      const int m = mb + kBlk * i;
      if (m >= g.M) continue;
      const int64_t off = static_cast<int64_t>(n) * ldc + m;
      const f32x4_t v = acc[i][j];
      if constexpr (kMode == static_cast<int>(EpiMode::kStoreF32)) {
        store4(static_cast<float*>(g.C) + split * g.split_stride + off, v);
      } else if constexpr (kMode == static_cast<int>(EpiMode::kAccumF32)) {
        store4(static_cast<float*>(g.C) + off, v);          // started from C's value
      } else if constexpr (kMode == static_cast<int>(EpiMode::kFinalOut)) {
        store4(static_cast<T*>(g.C) + off, v * osc);        // started from Cin's value
      } else if constexpr (kMode == static_cast<int>(EpiMode::kStoreOut)) {
        store4(static_cast<T*>(g.C) + off, v * csc[j]);
      } else if constexpr (kMode == static_cast<int>(EpiMode::kFinalAccum)) {
        T* c = static_cast<T*>(g.C) + off;
        store4(c, load4(c) + (load4(static_cast<const float*>(g.Cin) + off) + v) * osc);
      } else {
        T* c = static_cast<T*>(g.C) + off;
        store4(c, load4(c) + v * csc[j]);
      }
    }
  }
}

// ------------------------------------------------- logits + softmax stats
// Each wave reduces its own 128 classes (kStatCols): the statistics block of
// wave (wm) of tile tm is 2 tm + wm, so the epilogue needs no cross-wave
// exchange and no barrier.
static_assert(kWaveM == kStatCols, "one statistics block per wave");

// One logits tile (tm over classes, tn over chunk rows) with its epilogue.
// kRef: one reference per row (a.rref) instead of the block max.
template <typename T, bool kStoreT, bool kArgmax, bool kKTail, bool kRef>
__device__ __forceinline__ void logits_tile(const LogitsLse& a, int tm, int tn, char* lds) {
  static_assert(!kRef || kStoreT, "the per-row reference serves the gradient path");
  Acc acc;
  // M = classes (rows of W), N = chunk rows (rows of X), K = D.
  mainloop<T, kKTail, false, false>(static_cast<const T*>(a.W), a.ldw, tm * kTile, a.V, 0,
                                    static_cast<const T*>(a.X), a.ldx, tn * kTile, a.rows, 0,
                                    0, 0, a.D, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int c16 = lane & 15, q = lane >> 4;
  const int vbase = tm * kTile + wm * kWaveM;             // class of (i = 0, q = 0, r = 0)
  const int vlane = vbase + 4 * q;                        // + 16 i + r
  const int nbase = tn * kTile + wn * kWaveN + c16;       // chunk row of block j = 0
  const int64_t kblk = static_cast<int64_t>(vbase / kStatCols) * a.ldp;
  const T* bias = static_cast<const T*>(a.bias);
  const bool v_tail = vbase + kWaveM > a.V;               // uniform: classes past V in this wave

  // Targets (and references) of the lane's eight columns, fetched once
  // (-1: none / past the chunk).  A row past the chunk takes reference +inf,
  // so its T row is exp(-inf) = 0.
  int tcol[kJ];
  float rcol[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int n = nbase + kBlk * j;
    tcol[j] = n < a.rows ? a.tc[n] : -1;
    if constexpr (kRef) rcol[j] = n < a.rows ? a.rref[n] : INFINITY;
  }
  const int t_rows = kRef ? a.t_rows : a.rows;            // rows of T written

  // Bias of the lane's 32 classes, the same in all eight column blocks:
  // loaded once per tile, unconditionally, through a descriptor over
  // b[0 .. V), so that classes past V read 0.  One batch with the target
  // loads above (a per-element guarded load would wait on each).
  float bcol[kI][4] = {};
  if (bias) {                                             // uniform
    const __amdgpu_buffer_rsrc_t rbias =
        make_rsrc(bias, static_cast<int64_t>(a.V) * static_cast<int64_t>(sizeof(T)));
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        bcol[i][r] = load_elem<T>(rbias, (vlane + kBlk * i + r) * static_cast<int>(sizeof(T)));
  }

  // The epilogue walks the eight 16-column blocks j one at a time so that
  // only 32 accumulators per lane are live in VGPRs.
  // the tile's panel of T; the lane's first class within it
  T* Tm = static_cast<T*>(a.T) + static_cast<int64_t>(tm) * a.tps;
  const int vpan = wm * kWaveM + 4 * q;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    // Blocks not yet processed stay in the accumulator registers: without
    // this the register allocator copies every accumulator to VGPRs at the
    // loop exit and spills.
#pragma unroll
    for (int jj = j + 1; jj < kJ; ++jj)
#pragma unroll
      for (int i = 0; i < kI; ++i) asm volatile("" : "+a"(acc[i][jj]));
    // A block wholly past the rows of T (a short or ragged last chunk) has
    // nothing to store, and neither have the blocks after it.
    if (tn * kTile + wn * kWaveN + kBlk * j >= t_rows) break;   // uniform
    const int n = nbase + kBlk * j;         // chunk row
    const bool nin = n < a.rows;

    // 1. bias, and -inf for classes beyond V (both uniform branches).
    if (bias) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += bcol[i][r];
    }
    if (v_tail) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = vlane + kBlk * i + r < a.V ? acc[i][j][r] : -INFINITY;
    }

    // 2. target logit: the lane holding class tcol[j] of column n writes zt[n].
    {
      const int off = tcol[j] - vbase;
      if (tcol[j] >= 0 && off >= 0 && off < kWaveM && ((off >> 2) & 3) == q) {
        const int want = ((off >> 4) << 2) | (off & 3);
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < kI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) val = (i * 4 + r == want) ? acc[i][j][r] : val;
        a.zt[n] = val;
      }
    }

    // 3. column max (and lowest class attaining it) over the wave's 128
    //    classes: in-lane, then over the four lane groups of the column.
    float mx = -INFINITY;
    int mi = 0x7fffffff;
    if constexpr (kArgmax) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = acc[i][j][r];
          if (z > mx) {
            mx = z;
            mi = vlane + kBlk * i + r;
          }
        }
#pragma unroll
      for (int sh = 16; sh <= 32; sh <<= 1) {
        const float om = __shfl_xor(mx, sh);
        const int oi = __shfl_xor(mi, sh);
        if (om > mx || (om == mx && oi < mi)) {
          mx = om;
          mi = oi;
        }
      }
    } else {
      // max alone: fmaxf (NaN-skipping, as the comparison above) maps to
      // three-input maxima instead of a compare and a select per element
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[i][j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
    }

    // 4. e = exp(z - ref) in place, column sums; ref is the block max, or the
    //    row's reference.  A block wholly past V (max -inf) stores e = 0 and
    //    sum 0.
    const float ref = kRef ? rcol[j] : (mx == -INFINITY ? 0.0f : mx);
    const float nref = -ref * kLog2e;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // Block max: (z - max) first, so that the maximum maps to exactly 1
        // (a one-class row has loss exactly 0), which a fused
        // z log2(e) - max log2(e) would not give.  Row reference: no entry
        // needs to be exact (the combine forms the target entry from zt), so
        // one fused multiply-add forms the argument.
        const float x = kRef ? __builtin_fmaf(acc[i][j][r], kLog2e, nref)
                             : (acc[i][j][r] - ref) * kLog2e;
        const float e = __builtin_amdgcn_exp2f(x);
        acc[i][j][r] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);

    // 5. per-(row, statistics block) partials.
    if (nin && q == 0) {
      a.m_part[kblk + n] = mx;
      a.s_part[kblk + n] = sum;
      if constexpr (kArgmax) a.i_part[kblk + n] = mi;
    }
    if (kRef ? n < t_rows : nin) {
      // 6. the exp tile T[n][v]: 16-bit types trade halves between lane
      //    groups (pair_rows8) and store 8 consecutive classes at a time;
      //    fp32 stores 4.
      if constexpr (kStoreT) {
        T* row = Tm + static_cast<int64_t>(n) * kTile;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int p = 0; p < kI / 2; ++p)
            *reinterpret_cast<u32x4_t*>(row + wm * kWaveM + pair_off(p, q)) =
                pair_rows8<T>(acc[2 * p][j], acc[2 * p + 1][j]);
        } else {
#pragma unroll
          for (int i = 0; i < kI; ++i) store4(row + vpan + kBlk * i, acc[i][j]);
        }
      }
    }
    // keep the blocks apart so only one block's values are live at a time
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, bool kStoreT, bool kArgmax, bool kKTail, bool kRef>
__global__ __launch_bounds__(kThreads) void k_logits_lse(LogitsLse a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsOperandBytes];
  const int tiles_m = cdiv(a.V, kTile), tiles_n = cdiv(a.rows, kTile);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_coords(logical, tiles_m, tiles_n, 4, tm, tn);
  logits_tile<T, kStoreT, kArgmax, kKTail, kRef>(a, tm, tn, lds);
}

// The repair pass of the one-reference plan: nothing unless a flag is set
// (the common case costs one launch), else the tiles of the flagged rows
// again, shared evenly by a grid of at most one workgroup per CU.  Flag f
// covers gate_rows rows, whole 256-row tiles (0: one flag for all rows).
// The work items are (flagged row tile, class tile) pairs, numbered row
// tile by row tile; workgroup b takes items b, b + grid, ...  The flags are
// read by every wave of the workgroup alike, so the exits and the search
// for an item's row tile are uniform; each tile ends with the main loop's
// barrier, after which the LDS ring is free for the next tile.
template <typename T, bool kArgmax, bool kKTail>
__global__ __launch_bounds__(kThreads) void k_logits_repair(LogitsLse a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsOperandBytes];
  const int tiles_m = cdiv(a.V, kTile), tiles_n = cdiv(a.rows, kTile);
  const int per = a.gate_rows > 0 ? a.gate_rows / kTile : tiles_n;   // row tiles per flag
  const int nflags = cdiv(tiles_n, per);
  int flagged = 0;                                   // flagged row tiles
  for (int f = 0; f < nflags; ++f)
    if (a.gate[f]) flagged += min(per, tiles_n - f * per);
  const int items = flagged * tiles_m;
  for (int w = blockIdx.x; w < items; w += gridDim.x) {
    // the (w / tiles_m)-th flagged row tile, in row order
    int k = w / tiles_m, tn = 0;
    for (int f = 0; f < nflags; ++f) {
      if (!a.gate[f]) continue;
      const int cnt = min(per, tiles_n - f * per);
      if (k < cnt) {
        tn = f * per + k;
        break;
      }
      k -= cnt;
    }
    logits_tile<T, true, kArgmax, kKTail, true>(a, w % tiles_m, tn, lds);
  }
}

// Two entry points with the same body so profiles tell the products apart.
// grad_X's B is always T (panel layout, classes along K); grad_W's B is T
// when it is k-major, else the staged dL^T.
template <typename T, int kMode, bool kATr, bool kBTr>
__global__ __launch_bounds__(kThreads) void k_gemm_grad_x(GemmNT g) {
  gemm_nt_tile<T, kMode, kATr, kBTr, true>(g);
}
template <typename T, int kMode, bool kATr, bool kBTr>
__global__ __launch_bounds__(kThreads) void k_gemm_grad_w(GemmNT g) {
  gemm_nt_tile<T, kMode, kATr, kBTr, kBTr>(g);
}

// grad_W: every epilogue mode, B either the staged dL^T or T's panels (k-major).
template <typename T, bool kBTr>
void launch_grad_w(const GemmNT& g, dim3 grid, dim3 block, hipStream_t s) {
#define LCE_GEMM_CASE(mode)                                                                  \
  case EpiMode::mode:                                                                        \
    k_gemm_grad_w<T, static_cast<int>(EpiMode::mode), false, kBTr><<<grid, block, 0, s>>>(g); \
    break;
  switch (g.mode) {
    LCE_GEMM_CASE(kStoreF32)
    LCE_GEMM_CASE(kAccumF32)
    LCE_GEMM_CASE(kFinalOut)
    LCE_GEMM_CASE(kStoreOut)
    LCE_GEMM_CASE(kAccumOut)
    LCE_GEMM_CASE(kFinalAccum)
  }
#undef LCE_GEMM_CASE
}

// The layouts and modes the path uses, and no others:
//   grad_X: fp32 split partials (kStoreF32), or with one split and W read in
//           place the gradient itself (kStoreOut / kAccumOut); A = W^T
//           staged (fp32) or W read k-major in place (16-bit types); B = T's
//           panels, K-contiguous.
//   grad_W: any mode; A = X^T staged; B = the staged dL^T, or (16-bit types)
//           T's panels read k-major.
template <typename T>
hipError_t launch_gemm(const GemmNT& g, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>((g.M + kTile - 1) / kTile) *
                        ((g.N + kTile - 1) / kTile) * g.splits;
  if (tiles <= 0) return hipSuccess;
  if (tiles > INT32_MAX) return hipErrorInvalidValue;     // workgroup ids are int
  const dim3 grid(static_cast<uint32_t>(tiles)), block(kThreads);
  constexpr int kBK = kRowBytes / static_cast<int>(sizeof(T));
  // Every split range and K must be whole stages on this path.
  if (g.K % kBK != 0 || g.k_split % kBK != 0) return hipErrorInvalidValue;
  // B in the panel layout exactly where the kernel expects it.
  const bool pan = g.role == GemmRole::kGradX || g.b_kmajor;
  if (pan != (g.b_pstride > 0) || (pan && g.ldb != kTile)) return hipErrorInvalidValue;
  // Column factors only where the epilogue applies them.
  if (g.n_scale && g.mode != EpiMode::kStoreOut && g.mode != EpiMode::kAccumOut)
    return hipErrorInvalidValue;
  constexpr bool k16 = sizeof(T) == 2;
  if (g.role == GemmRole::kGradX) {
    // fp32 split partials; or, for 16-bit types reading W in place with one
    // split, grad_X itself (stored or added, in the element type).
    const bool direct = g.mode == EpiMode::kStoreOut || g.mode == EpiMode::kAccumOut;
    if (g.b_kmajor || (g.a_kmajor && !k16)) return hipErrorInvalidValue;
    if (g.mode != EpiMode::kStoreF32 && !(direct && k16 && g.a_kmajor && g.splits == 1))
      return hipErrorInvalidValue;
    if constexpr (k16) {
      if (g.a_kmajor) {
        if (g.mode == EpiMode::kStoreOut)
          k_gemm_grad_x<T, static_cast<int>(EpiMode::kStoreOut), true, false>
              <<<grid, block, 0, s>>>(g);
        else if (g.mode == EpiMode::kAccumOut)
          k_gemm_grad_x<T, static_cast<int>(EpiMode::kAccumOut), true, false>
              <<<grid, block, 0, s>>>(g);
        else
          k_gemm_grad_x<T, static_cast<int>(EpiMode::kStoreF32), true, false>
              <<<grid, block, 0, s>>>(g);
        return hipGetLastError();
      }
    }
    k_gemm_grad_x<T, static_cast<int>(EpiMode::kStoreF32), false, false><<<grid, block, 0, s>>>(g);
    return hipGetLastError();
  }
  // grad_W.  Both operands k-major doubles the transposing LDS reads per MFMA
  // and measured slower than staging one of them; it is not built.
  if (g.a_kmajor || (g.b_kmajor && !k16)) return hipErrorInvalidValue;
  if constexpr (k16) {
    if (g.b_kmajor) {
      launch_grad_w<T, true>(g, grid, block, s);
      return hipGetLastError();
    }
  }
  launch_grad_w<T, false>(g, grid, block, s);
  return hipGetLastError();
}

template <typename T, bool kKTail>
void launch_logits_k(const LogitsLse& a, dim3 grid, dim3 block, hipStream_t s) {
  const bool st = a.T != nullptr, am = a.i_part != nullptr;
  if constexpr (std::is_same_v<T, uint16_t>) {
    if (a.rref) {
      if (a.gate) {
        grid.x = std::min<uint32_t>(grid.x, kRepairGrid);
        if (am) k_logits_repair<T, true, kKTail><<<grid, block, 0, s>>>(a);
        else k_logits_repair<T, false, kKTail><<<grid, block, 0, s>>>(a);
      } else if (am) {
        k_logits_lse<T, true, true, kKTail, true><<<grid, block, 0, s>>>(a);
      } else {
        k_logits_lse<T, true, false, kKTail, true><<<grid, block, 0, s>>>(a);
      }
      return;
    }
  }
  if (st && am) k_logits_lse<T, true, true, kKTail, false><<<grid, block, 0, s>>>(a);
  else if (st) k_logits_lse<T, true, false, kKTail, false><<<grid, block, 0, s>>>(a);
  else if (am) k_logits_lse<T, false, true, kKTail, false><<<grid, block, 0, s>>>(a);
  else k_logits_lse<T, false, false, kKTail, false><<<grid, block, 0, s>>>(a);
}

template <typename T>
hipError_t launch_logits(const LogitsLse& a, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>((a.V + kTile - 1) / kTile) *
                        ((a.rows + kTile - 1) / kTile);
  if (tiles <= 0) return hipSuccess;
  if (tiles > INT32_MAX) return hipErrorInvalidValue;     // workgroup ids are int
  // The per-row reference: bf16 with T only; rows of T between rows and
  // t_rows stay inside the chunk's last tile row; the repair needs the flag.
  if (a.rref && (!std::is_same_v<T, uint16_t> || a.T == nullptr || a.t_rows < a.rows ||
                 static_cast<int64_t>(a.t_rows) > ((a.rows + kTile - 1) / kTile) * kTile))
    return hipErrorInvalidValue;
  if (a.gate && (!a.rref || a.gate_rows < 0 || a.gate_rows % kTile != 0))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(tiles)), block(kThreads);
  constexpr int kBK = kRowBytes / static_cast<int>(sizeof(T));
  if (a.D % kBK == 0) launch_logits_k<T, false>(a, grid, block, s);
  else launch_logits_k<T, true>(a, grid, block, s);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_nt(Elem e, const GemmNT& g, hipStream_t s) {
  if (e == Elem::kBF16) return launch_gemm<uint16_t>(g, s);
  if (e == Elem::kF16) return launch_gemm<_Float16>(g, s);
  return launch_gemm<float>(g, s);
}

hipError_t logits_lse(Elem e, const LogitsLse& a, hipStream_t s) {
  if (e == Elem::kBF16) return launch_logits<uint16_t>(a, s);
  if (e == Elem::kF16) return launch_logits<_Float16>(a, s);
  return launch_logits<float>(a, s);
}

}  // namespace lce
