// Direct global -> LDS staging used by the LDS-pipelined GEMM kernels.
#pragma once

#include "common.h"

namespace qg {

typedef __attribute__((address_space(3))) void lds_void_t;

// global_load_lds_dwordx4: 16 bytes per lane from global memory straight into
// LDS; lane l writes lds_base + 16*l (lds_base is wave-uniform, passed in M0).
// The global address needs only 2-byte alignment (checked on gfx950).
// Issued from inline assembly on purpose: the compiler does not count these
// loads, so it adds no wait for them before every LDS read (it cannot tell
// the stage being filled from the one being read); the kernels wait for them
// with an explicit vmcnt and a barrier.
// The compiler's hazard tracking does not look inside the assembly either, so
// the statement opens with the wait states the load needs after the
// instructions that set up its operands: 5 after a VALU write of an SGPR it
// reads (the base address arrives through v_readfirstlane), 1 after an SALU
// write of M0.  Without them the load could read a stale base register and
// fetch from an arbitrary address.
#define QG_LDS_DMA_WAIT "s_nop 4\n\t"
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds_dst)));
  asm volatile(QG_LDS_DMA_WAIT "global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same load with a wave-uniform 64-bit base in SGPRs and a per-lane
// 32-bit byte offset (the saddr form): address = base + voff.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ void lds_dma16_sv(const void* base, uint32_t voff, const void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds_dst)));
  asm volatile(QG_LDS_DMA_WAIT "global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)), "{m0}"(m0)
               : "memory");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS reads are done, then meet the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}


}  // namespace qg
