// Loads that write LDS directly, and the waits and barriers around them, for
// gfx950.
//
// buffer_load_dwordx4 ... lds writes each lane's 16 bytes to LDS at
// M0 + 16 * lane: one instruction fills 1 KB of LDS contiguously, and the
// lane's global address is free, so a swizzled LDS layout is built by choosing
// which global chunk each lane fetches.  An offset at or past the descriptor's
// num_records returns zeros without touching memory; that masks rows and the
// k tail without a branch.  These loads count in vmcnt only.
//
// They are issued through inline assembly and every wait is placed by hand:
// the compiler's own bookkeeping would treat each LDS read as dependent on
// every load into LDS still in flight and drain them all before it.
#pragma once

#include "common.h"

namespace fmlp {

constexpr uint32_t kOutOfRange = 0x80000000u;  // offset past any descriptor's end

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  compiler_fence();
}
// Workgroup barrier for LDS hand-off: this wave's LDS accesses are complete,
// then all waves meet.  No vector-memory wait: loads into LDS are waited for
// explicitly, per stage, before it.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Every descriptor here is wave-uniform by construction; readfirstlane puts it
// in SGPRs so no load needs a per-lane loop.  readfirstlane returns a signed
// int: each half is widened through uint32_t, never sign-extended into the
// other.
__device__ __forceinline__ uint32_t uniform32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
// raw buffer descriptor in SGPRs: base, stride 0, num_records = bytes
__device__ __forceinline__ i32x4_t make_desc(uint64_t base, uint32_t bytes) {
  i32x4_t d;
  d[0] = (int)uniform32((uint32_t)base);
  d[1] = (int)(uniform32((uint32_t)(base >> 32)) & 0xFFFFu);
  d[2] = (int)uniform32(bytes);
  d[3] = 0x00020000;
  return d;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uniform32((uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane into LDS at lds + 16 * lane (lds wave-uniform)
__device__ __forceinline__ void asm_load_lds(const i32x4_t& d, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(off), "s"(d), "s"(lds) : "memory", "m0");
}
// the same for data read exactly once (a weight stream): the non-temporal
// policy keeps it from displacing reused lines in L2 and the Infinity Cache
__device__ __forceinline__ void asm_load_lds_stream(const i32x4_t& d, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(off), "s"(d), "s"(lds) : "memory", "m0");
}
// the same with a wave-uniform byte offset soff added to every lane's offset
__device__ __forceinline__ void asm_load_lds(const i32x4_t& d, uint32_t lds, uint32_t off,
                                             uint32_t soff) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :: "v"(off), "s"(d), "s"(lds), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace fmlp
