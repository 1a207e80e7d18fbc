// Device helpers shared by the kernel translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {
namespace dev {

// Raw buffer descriptor (gfx9 layout: base, stride 0, byte range, dword3 =
// 0x00020000).  Loads whose per-lane offset is at or past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int range = bytes > 0x7ffff000LL * 2 ? -1 : static_cast<int>(static_cast<uint32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, range, 0x00020000);
}
constexpr int kOutOfRange = 0x7fffffff;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}

// One 16-byte-per-lane copy from a buffer straight into LDS at `lds` (M0) +
// 16 * lane; the global address is base + voffset + soffset.  Issued as
// inline asm so the compiler does not track it: its waits for LDS copies
// would cover every copy in flight (including ones issued for later use).
// Callers wait for the copies themselves; vector memory operations complete
// in issue order, so any wait the compiler inserts for its own loads stays
// correct (at worst stronger than needed).  The s_nop is the wait state the
// ISA asks for between an SALU write of M0 and an LDS-DMA read of it.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, int voffset,
                                              uint32_t lds, int soffset = 0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory");
}

// gfx9 s_waitcnt immediates: vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; expcnt and lgkmcnt at their maxima mean "do not wait".
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

}  // namespace dev
}  // namespace lce
