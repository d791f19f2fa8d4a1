// Direct global->LDS copies (global_load_lds_dwordx4) shared by the kernels that
// stream K/V tiles into LDS rings: the union decode, the dense decode and the
// query-tile prefill.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace msa {

// s_waitcnt immediate (gfx9 encoding): vmcnt <= n (n < 16) together with lgkmcnt(0)
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4); }

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
}

// One 16-byte direct global->LDS load per lane: lane l's 16 bytes from `src` land
// at LDS byte lds_base + 16 l (lds_base wave-uniform, in M0). Written as inline
// assembly so that the compiler does not track it: its own waits for these loads
// would otherwise cover every buffer of a ring before any LDS read. Completion is
// waited for by hand with vmcnt (loads retire in issue order), and the memory
// clobber keeps LDS accesses from moving across the load.
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base) : "memory");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (address = base + offset), so that per-lane address arithmetic stays
// 32-bit and loop-invariant.
__device__ __forceinline__ void lds_load16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_base)
               : "memory");
}

// The same two copies with the non-temporal hint, for K/V streamed once (the decode
// kernels: 5% faster on the union decode, 2% on the dense decode, same bits).
__device__ __forceinline__ void lds_load16_nt(const void* src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_load16_s_nt(const void* sbase, uint32_t voff,
                                                uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "{m0}"(lds_base)
               : "memory");
}

}  // namespace msa
