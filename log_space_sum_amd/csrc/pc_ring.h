// pc_ring.h -- the pieces of the products' LDS rings: direct global->LDS
// loads issued from inline assembly (so the compiler, which cannot tell the
// ring's stages apart, does not drain every load in flight before each LDS
// read), explicit vector-memory waits, and a barrier without a memory fence.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pc {

// One 16-byte direct global->LDS load per lane: lane L writes LDS bytes
// [m0 + 16 L, m0 + 16 L + 16) from sbase + voff.  Issued from inline assembly:
// the ring tracks its completion with explicit vmcnt waits, and a compiler
// that cannot tell the stages apart would otherwise drain every in-flight
// load before each LDS read.  (M0, the LDS base of the instruction, has no
// other user in these kernels.)
__device__ __forceinline__ void lds_load16(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte);
  // the base is uniform: pin it to scalar registers (readfirstlane returns a
  // signed int, so each half goes through uint32_t before widening)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t sb = (hi << 32) | lo;
  // one wait state between the SALU write of M0 and the LDS DMA reading it
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(m0)
               : "memory", "m0");
}

// s_waitcnt immediate: at most `vm` vector-memory operations outstanding, no
// LDS operation outstanding (expcnt left at its maximum).
template <int vm>
struct WaitVmLgkm {
  static_assert(vm >= 0 && vm <= 63, "vmcnt is a 6-bit counter");
  static constexpr int imm = (vm & 15) | ((vm >> 4) << 14) | (7 << 4);
};

// Workgroup barrier without a memory fence (the ring's loads stay in flight);
// the signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 4-byte direct global->LDS load per active lane: lane L writes LDS bytes
// [m0 + 4 L, m0 + 4 L + 4) from sbase + voff (inactive lanes write nothing).
__device__ __forceinline__ void lds_load4(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t sb = (hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sb), "s"(m0)
               : "memory", "m0");
}

}  // namespace pc
