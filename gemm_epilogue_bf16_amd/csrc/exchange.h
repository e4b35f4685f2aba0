// Device helpers of the cross-block exchange inside one launch (the decode
// engines publish a layer's output and every block gathers it), for gfx950:
// device-coherent loads and stores of the exchanged words and flags, and the
// epoch that tags one call's words.
#pragma once

#include "common.h"
#include "lds_dma.h"

namespace fmlp {

__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent (sc1) stores of h through a buffer descriptor.  A buffer
// store counts in vmcnt only; a store through a generic pointer would be a
// flat store, which also holds lgkmcnt until it completes and so stalls the
// next LDS wait of the storing wave behind a write-through to memory.  The
// 16-byte form writes two 8-byte words, each whole.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_coherent_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ void st_coherent_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t ua = ((uint64_t)uniform32((uint32_t)(a >> 32)) << 32) | (uint64_t)uniform32((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ua), (short)0,
                                           (int)uniform32(bytes), 0x00020000);
}
// The epoch of a call: generation g (odd multiplier: distinct g give distinct
// values) plus the launch's salt; never 0, the value of a zeroed flag.
__device__ __forceinline__ uint32_t epoch_of(uint32_t g, uint32_t salt) {
  const uint32_t e = g * 0x9E3779B1u + salt;
  return e ? e : 1u;
}

}  // namespace fmlp
